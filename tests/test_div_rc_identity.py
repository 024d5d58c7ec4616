"""The AdamW kernels divide by a float32 c through the float64 reciprocal:
fl32(fl64(x * fl64(1 / c))). For every float32 x and positive float32 c this
equals the correctly rounded float32 quotient fl32(x / c) (a quotient of two
float32 values lies more than 2^-49 relative from every float32 midpoint,
the float64 product within 2^-52 of it). Checked here with numpy's IEEE
arithmetic on random pairs over the whole exponent range, on divisors with
all-ones and single-bit mantissas, and on dividends that are exact
multiples of the divisor or land next to midpoints."""

import numpy as np


def _via_rc(x, c):
    rc = 1.0 / c.astype(np.float64)
    return (x.astype(np.float64) * rc).astype(np.float32)


def _check(x, c):
    with np.errstate(over="ignore", under="ignore", divide="ignore", invalid="ignore"):
        want = (x / c).astype(np.float32)
        got = _via_rc(x, c)
    same = (want.view(np.uint32) == got.view(np.uint32)) | (np.isnan(want) & np.isnan(got))
    assert same.all(), (x[~same][:4], c[~same][:4])


def test_random_pairs_all_exponents():
    rng = np.random.default_rng(0)
    n = 2_000_000
    x = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32).view(np.float32)
    c = (rng.integers(1, 0x7F800000, n, dtype=np.uint64).astype(np.uint32)).view(np.float32)
    keep = np.isfinite(x)
    _check(x[keep], c[keep])


def test_optimizer_ranges():
    """Moments, bias corrections and block scales of the magnitudes the
    optimizer sees."""
    rng = np.random.default_rng(1)
    n = 2_000_000
    x = (rng.standard_normal(n) * np.exp(rng.uniform(-60, 5, n))).astype(np.float32)
    for c in (np.float32(1 - 0.9), np.float32(1 - 0.999), np.float32(1 - 0.999 ** 7),
              np.float32(1 - 0.9 ** 1000), np.float32(3e-4 / 448), np.float32(1e-9 / 57344)):
        _check(x, np.full(n, c, np.float32))
    c = np.abs(rng.standard_normal(n) * np.exp(rng.uniform(-40, 0, n))).astype(np.float32)
    c[c == 0] = 1.0
    _check(x, c)


def test_structured_divisors_and_dividends():
    rng = np.random.default_rng(2)
    exps = np.arange(-140, 128, 7, dtype=np.int64)
    mant_all_ones = np.full(exps.size, (1 << 23) - 1, np.int64)
    cs = []
    for mant in (mant_all_ones, np.zeros(exps.size, np.int64), np.full(exps.size, 1, np.int64),
                 np.full(exps.size, (1 << 22) | 1, np.int64)):
        bits = ((np.clip(exps + 127, 1, 254) << 23) | mant).astype(np.uint32)
        cs.append(bits.view(np.float32))
    cs = np.concatenate(cs)
    for c in cs:
        # exact multiples q * c, their neighbours, and values next to q.5 * c
        q = rng.integers(1, 1 << 24, 4096).astype(np.float32)
        with np.errstate(over="ignore", under="ignore"):
            base = (q * c).astype(np.float32)
            mid = ((q + np.float32(0.5)) * c).astype(np.float32)
        xs = [base, np.nextafter(base, np.float32(np.inf)), np.nextafter(base, np.float32(0)),
              mid, np.nextafter(mid, np.float32(np.inf)), np.nextafter(mid, np.float32(0))]
        x = np.concatenate(xs)
        x = x[np.isfinite(x)]
        _check(x, np.full(x.size, c, np.float32))
