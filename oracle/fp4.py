"""The FP4 4-bit data type as a 16-entry codebook (TEST INFRASTRUCTURE ONLY).

The pages name FP4 only as the 4-bit alternative to NF4 that one should not
pick without a reason ([P4] "Common mistakes"), and do not define it.
Reading: FP4 is the OCP MX E2M1 format (one sign bit, two exponent bits,
one mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), scaled by 1/6 so
that, like NF4, its range is [-1, 1] with an exact 0 and exact endpoints.

Codes are sign-magnitude, as in E2M1: code = 8 s + m, value (-1)^s E2M1(m)/6,
so code 8 is -0 (equal to 0). Levels are the float32 roundings of these
exact rationals (1/12, 1/6, 1/3, 2/3 are not exact in float32).

Nearest level of a float32 n (|n| <= 1, n = w / c as for NF4): the code
whose level is at the least exact distance; among codes at the same
distance, the one with an even magnitude m (the E2M1 rule: ties to the
even mantissa), then the lower code (so 0 maps to +0, code 0; code 8 is
never produced). An all-zero block stores code 0.

Ties: the only midpoints of adjacent float32 levels that are themselves
float32 numbers are those between 0 and +-1/12; there n goes to 0.

Pinned by the exact rational values (from the E2M1 bit layout) and their
float32 roundings, sign symmetry, a brute force over every code with exact
rational distances at every float32 next to each decision point, the E2M1
round-to-nearest-even conversion of the exact 6 n away from decision points,
the two ties, and the round-trip error bound.
"""

from fractions import Fraction

import numpy as np

# E2M1 magnitudes (exponent bias 1; m = 1 is the subnormal 0.5)
E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
        Fraction(4), Fraction(6)]
ZERO_CODE = 0


def levels_exact():
    """The 16 levels in code order as exact rationals."""
    out = []
    for c in range(16):
        s, m = c >> 3, c & 7
        v = E2M1[m] / 6
        out.append(-v if s else v)
    return out


def codebook():
    """The 16 levels in code order, each the correctly rounded float32 of
    its exact value (code 8 is -0.0)."""
    out = np.empty(16, dtype=np.float32)
    for c, v in enumerate(levels_exact()):
        out[c] = _round_f32(v)
    out[8] = np.float32(-0.0)
    return out


def _round_f32(v):
    """Correctly rounded float32 of an exact rational (nearest, ties even)."""
    f = np.float32(float(v))
    # candidates around f; pick the nearest exactly
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = None
    for c in cands:
        d = abs(Fraction(float(c)) - v)
        key = (d, int(np.float32(c).view(np.uint32)) & 1)  # ties: even significand
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def nearest_code(n, levels=None):
    """FP4 code of each float32 value n: least exact distance, ties to the
    even magnitude, then to the lower code. Distances are taken in float64,
    which is exact for the difference of two float32 values of this range."""
    if levels is None:
        levels = codebook()
    n64 = np.asarray(n, dtype=np.float32).astype(np.float64)
    lv = np.asarray(levels, dtype=np.float32).astype(np.float64)
    dist = np.abs(n64[..., None] - lv)
    # preference key: distance first, then odd magnitude after even, then code
    codes = np.arange(16)
    rank = (codes & 1) * 16 + codes          # even magnitude first, then lower code
    order = np.argsort(rank, kind="stable")  # codes in preference order
    d_ord = dist[..., order]
    pick = np.argmin(d_ord, axis=-1)         # first minimum in preference order
    return order[pick].astype(np.uint8)
