"""Pins for the oracle's NF4 codebook (CPU only).

The codebook is fixed by the pages as 16 levels at normal quantiles with
equal probability mass per bin, scaled into [-1, 1], and by the invariants
the type must keep (exact zero, endpoints -1 and +1). Each check below would
fail for a plausible slip in the construction: a symmetric split, a missing
zero, a wrong normalization, a swapped half, an off-by-one in the
probability grid, or a wrong inverse CDF.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import nf4


def _bisect_inv_cdf(p):
    """Independent normal quantile: bisection on Phi(x) = erfc(-x/sqrt2)/2."""
    lo, hi = -40.0, 40.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if mid == lo or mid == hi:
            break
        if 0.5 * math.erfc(-mid / math.sqrt(2.0)) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def _phi(x):
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def check_codebook(levels64, levels32):
    """All codebook invariants; returns a list of failures (empty = pass)."""
    fails = []
    if levels32.shape != (16,):
        return ["not 16 levels"]
    if not np.all(np.diff(levels32.astype(np.float64)) > 0):
        fails.append("levels not strictly increasing")
    if levels32[0] != np.float32(-1.0) or levels32[15] != np.float32(1.0):
        fails.append("endpoints not exactly -1 and +1")
    if levels32[7] != np.float32(0.0):
        fails.append("no exact zero at index 7")
    # equal mass per bin within each half: map the levels back to
    # probabilities through Phi and check the grid spacing.
    top = _bisect_inv_cdf(nf4.P_MAX)
    probs = np.array([_phi(v * top) for v in levels64])
    pos = probs[8:]
    neg = 1.0 - probs[:7][::-1]
    step_pos = (nf4.P_MAX - 0.5) / 8
    step_neg = (nf4.P_MAX - 0.5) / 7
    if not np.allclose(np.diff(np.concatenate([[0.5], pos])), step_pos, rtol=0, atol=1e-12):
        fails.append("positive bins do not hold equal mass")
    if not np.allclose(np.diff(np.concatenate([[0.5], neg])), step_neg, rtol=0, atol=1e-12):
        fails.append("negative bins do not hold equal mass")
    # the mass of every bin is the same fraction of its half
    if abs(pos[-1] - nf4.P_MAX) > 1e-12 or abs(neg[-1] - nf4.P_MAX) > 1e-12:
        fails.append("outermost levels not at the truncation probability")
    return fails


def test_codebook_invariants():
    assert check_codebook(nf4.codebook_fp64(), oracle.codebook()) == []


def test_codebook_independent_inverse_cdf_bitwise():
    a = nf4.codebook_fp64().astype(np.float32)
    b = nf4.codebook_fp64(inv_cdf=_bisect_inv_cdf).astype(np.float32)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_codebook_levels_far_from_float32_ties():
    """Every level is far from a float32 rounding tie, so any accurate
    inverse CDF rounds to the same bits."""
    l64 = nf4.codebook_fp64()
    for v in l64:
        if v == 0.0 or abs(v) == 1.0:
            continue
        f = np.float32(v)
        ulp = float(np.spacing(np.float32(abs(f))))
        frac = abs(v - float(f)) / ulp
        assert frac < 0.5 - 1e-6, (v, frac)


def test_codebook_p_max_value():
    assert nf4.P_MAX_FRACTION == nf4.Fraction(929, 960)
    assert abs(nf4.P_MAX - 0.9677083333333333) < 1e-16


def test_level8_exact():
    l8 = oracle.level8()
    assert l8[0] == 0 and l8[255] == 1
    for k in range(256):
        # correctly rounded k/255: the float32 nearest to the rational
        exact = nf4.Fraction(k, 255)
        f = nf4.Fraction(float(l8[k]))
        up = nf4.Fraction(float(np.nextafter(l8[k], np.float32(2))))
        dn = nf4.Fraction(float(np.nextafter(l8[k], np.float32(-1))))
        assert abs(f - exact) <= abs(up - exact) and abs(f - exact) <= abs(dn - exact)


# --- planted mistakes: each must be caught by check_codebook ---------------

def _symmetric_no_zero():
    # 16 quantiles at (i + 1/2)/16: no exact zero, no +-1
    from statistics import NormalDist
    nd = NormalDist()
    v = np.array([nd.inv_cdf((i + 0.5) / 16) for i in range(16)])
    v = v / v[-1]
    return v


def _swapped_halves():
    l = nf4.codebook_fp64().copy()
    return np.sort(-l)


def _uniform_levels():
    return np.concatenate([np.linspace(-1, 0, 8), np.linspace(0, 1, 9)[1:]])


@pytest.mark.parametrize("maker", [_symmetric_no_zero, _swapped_halves, _uniform_levels])
def test_planted_codebook_mistakes_are_caught(maker):
    l64 = np.asarray(maker(), dtype=np.float64)
    assert check_codebook(l64, l64.astype(np.float32)) != []
