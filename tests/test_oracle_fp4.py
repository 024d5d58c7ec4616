"""Pins of the FP4 codebook, its nearest-code rule and the stored types that
use it or the 8-bit floating-point constant code (oracle.fp4, oracle.store)."""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import fp4, fp8, store


def _e2m1_from_bits(m):
    """E2M1 magnitude of the 3-bit field m (exponent bits 2-1, mantissa bit
    0, exponent bias 1; exponent 0 is subnormal), from the format's layout."""
    e, f = m >> 1, m & 1
    if e == 0:
        return Fraction(f, 2)
    return Fraction(2) ** (e - 1) * (1 + Fraction(f, 2))


def test_levels_are_e2m1_over_six():
    lv = fp4.codebook()
    assert lv.dtype == np.float32 and lv.size == 16
    for c in range(16):
        exact = _e2m1_from_bits(c & 7) / 6 * (-1 if c >> 3 else 1)
        got = Fraction(float(lv[c]))
        ulp = Fraction(float(np.spacing(np.float32(abs(float(exact))) or np.float32(1e-30))))
        assert abs(got - exact) <= ulp / 2, (c, float(got), float(exact))
    # exact endpoints and zero; symmetric; 15 distinct values
    assert lv[7] == 1.0 and lv[15] == -1.0 and lv[0] == 0.0 and lv[8] == 0.0
    assert np.signbit(lv[8]) and not np.signbit(lv[0])
    assert np.array_equal(lv[8:], -lv[:8])
    assert len(set(lv.tolist())) == 15
    # exactly representable levels are exact
    for c, v in ((3, 0.25), (5, 0.5), (7, 1.0)):
        assert lv[c] == np.float32(v)


def _brute(n):
    """Nearest code by exact rational distances; ties: even magnitude, then
    lower code (a plain loop over the 16 codes)."""
    lv = fp4.codebook()
    x = Fraction(float(n))
    best = None
    for c in range(16):
        d = abs(x - Fraction(float(lv[c])))
        key = (d, c & 1, c)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def _decision_points():
    lv = np.unique(fp4.codebook().astype(np.float64))
    return [(lv[i] + lv[i + 1]) / 2 for i in range(len(lv) - 1)]


def test_nearest_code_brute_force_at_every_decision_point():
    pts = []
    for mid in _decision_points():
        f = np.float32(mid)
        for k in range(-3, 4):
            g = f
            for _ in range(abs(k)):
                g = np.nextafter(g, np.float32(np.inf if k > 0 else -np.inf))
            pts.append(g)
    pts += list(np.float32([-1.0, 1.0, 0.0, -0.0]))
    pts = np.array(pts, dtype=np.float32)
    got = fp4.nearest_code(pts)
    want = np.array([_brute(p) for p in pts])
    assert np.array_equal(got, want)


def test_nearest_code_brute_force_random():
    rng = np.random.default_rng(7)
    n = np.concatenate([rng.uniform(-1, 1, 3000), rng.uniform(-0.1, 0.1, 1000)]).astype(np.float32)
    assert np.array_equal(fp4.nearest_code(n), [_brute(x) for x in n])


def test_tie_rule_on_representable_midpoints():
    """Where the midpoint of two adjacent levels is a float32, it takes the
    code with the even magnitude (the E2M1 rounding rule); zero takes +0."""
    lv = fp4.codebook()
    found = 0
    for mid in _decision_points():
        f = np.float32(mid)
        if float(f) != mid:
            continue
        found += 1
        c = int(fp4.nearest_code(np.array([f]))[0])
        assert (c & 1) == 0, (mid, c)
        lo = max(x for x in lv.astype(np.float64) if x < mid)
        hi = min(x for x in lv.astype(np.float64) if x > mid)
        assert float(lv[c]) in (lo, hi)
    # 0 | 1/12 and -1/12 | 0 are the only midpoints of adjacent float32
    # levels that are float32 numbers (the others need a 25th bit), so these
    # are the only ties the rule ever decides: both go to 0
    assert found == 2
    assert int(fp4.nearest_code(np.float32([0.0]))[0]) == 0
    assert int(fp4.nearest_code(np.float32([-0.0]))[0]) == 0


def _e2m1_rne_code(n):
    """Code of the E2M1 value nearest to the exact rational 6 n, ties to the
    even mantissa (the format's own conversion), for |6 n| <= 6."""
    x = Fraction(float(n)) * 6
    mags = [_e2m1_from_bits(m) for m in range(8)]
    best = min(range(8), key=lambda m: (abs(abs(x) - mags[m]), m & 1))
    return best if (x >= 0 or best == 0) else 8 + best


def test_agrees_with_e2m1_conversion_of_6n():
    """Away from decision points (where the float32 rounding of 1/12, 1/6,
    1/3 and 2/3 could matter), the nearest float32 level is the E2M1 value
    that the format's round-to-nearest-even conversion gives for 6 n."""
    rng = np.random.default_rng(13)
    n = rng.uniform(-1, 1, 4000).astype(np.float32)
    mids = np.array(_decision_points())
    far = np.min(np.abs(n.astype(np.float64)[:, None] - mids[None, :]), axis=1) > 1e-6
    got = fp4.nearest_code(n[far])
    want = np.array([_e2m1_rne_code(x) for x in n[far]])
    assert far.sum() > 3900 and np.array_equal(got, want)


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy()


@pytest.mark.parametrize("st", [1, 3])
def test_fp4_store_round_trip_bound(st):
    """|w - w'| <= c * 1/6 + |L| |c - c'|: the largest half gap between FP4
    levels is (1 - 2/3) / 2; the block maximum maps to +-1."""
    rng = np.random.default_rng(st)
    w = _bf16(rng.standard_t(5, 64 * 300) * 0.02)
    r = store.quantize(w, st)
    wp = store.dequantize(r["codes"], r["absmax_q"], r["absmax_s2"], w.size, st)
    c = r["absmax"][np.arange(w.size) // 64].astype(np.float64)
    cp = store.block_constants(r["absmax_q"], r["absmax_s2"], st)[np.arange(w.size) // 64]
    lv = store.levels(st)[r["q"]].astype(np.float64)
    bound = c / 6 + np.abs(lv) * np.abs(c - cp) + 1e-12
    assert np.all(np.abs(w - wp) <= bound)
    blocks = w.reshape(-1, 64)
    am = np.argmax(np.abs(blocks), axis=1)
    qb = r["q"].reshape(-1, 64)[np.arange(len(am)), am]
    sign = blocks[np.arange(len(am)), am] < 0
    assert np.array_equal(qb, np.where(sign, 15, 7))


def test_fp4_zero_block_and_codes_never_negative_zero():
    w = np.zeros(130, np.float32)
    w[70] = 0.5
    w[71] = -1e-3
    r = store.quantize(w, 1)
    assert np.all(r["q"][:64] == 0)
    assert 8 not in r["q"].tolist()


def test_type_zero_is_the_nf4_oracle():
    rng = np.random.default_rng(3)
    w = _bf16(rng.standard_normal(64 * 700 + 17) * 0.02)
    a, b = store.quantize(w, 0), oracle.quantize(w)
    for k in ("codes", "absmax_q", "absmax_s2"):
        assert np.array_equal(a[k], b[k])
    da = store.dequantize(a["codes"], a["absmax_q"], a["absmax_s2"], w.size, 0)
    db = oracle.dequantize(b["codes"], b["absmax_q"], b["absmax_s2"], w.size)
    assert np.array_equal(da.view(np.uint32), db.view(np.uint32))


@pytest.mark.parametrize("st", [2, 3])
def test_fp8_constant_code_against_torch_float8(st):
    """The second level of the 8-bit floating-point code: S = fl32(max / 448)
    per group, q8 the E4M3 code of fl32(c / S), as torch's float8_e4m3fn
    conversion gives it (values above 448 saturate to 448)."""
    rng = np.random.default_rng(11 + st)
    w = _bf16(rng.standard_t(5, 64 * 256 * 3 + 64 * 10) * 0.02)
    r = store.quantize(w, st)
    nb = r["absmax"].size
    g = np.arange(nb) // 256
    S = r["absmax_s2"]
    gmax = np.array([r["absmax"][g == k].max() for k in range(S.size)], np.float32)
    assert np.array_equal(S.view(np.uint32), (gmax / np.float32(448.0)).astype(np.float32).view(np.uint32))
    ratio = (r["absmax"] / S[g]).astype(np.float32)
    t = torch.from_numpy(np.minimum(ratio, np.float32(448.0))).to(torch.float8_e4m3fn)
    assert np.array_equal(r["absmax_q"], t.view(torch.uint8).numpy())
    # the group maximum decodes to about the group maximum
    cp = store.block_constants(r["absmax_q"], S, st)
    for k in range(S.size):
        i = np.flatnonzero(g == k)[np.argmax(r["absmax"][g == k])]
        assert abs(float(cp[i]) - float(r["absmax"][i])) <= 2.0 ** -4 * float(r["absmax"][i])


def test_fp8_constant_code_relative_half_step():
    """|c - c'| <= 2^-4 c + rounding, for every constant at least 2^-6 of its
    group maximum (normal E4M3 range relative to 448 S)."""
    rng = np.random.default_rng(5)
    w = _bf16(rng.standard_t(3, 64 * 256 * 4) * 0.02)
    r = store.quantize(w, 2)
    g = np.arange(r["absmax"].size) // 256
    c = r["absmax"].astype(np.float64)
    cp = store.block_constants(r["absmax_q"], r["absmax_s2"], 2).astype(np.float64)
    big = c >= 2.0 ** -6 * 448.0 * r["absmax_s2"][g]
    assert big.sum() > 500
    assert np.all(np.abs(c - cp)[big] <= 2.0 ** -4 * c[big] * (1 + 2.0 ** -20))


def test_fp8_zero_group():
    w = np.zeros(64 * 256 * 2, np.float32)
    w[64 * 256 + 5] = 0.25
    r = store.quantize(w, 2)
    assert r["absmax_s2"][0] == 0 and np.all(r["absmax_q"][:256] == 0)
    wp = store.dequantize(r["codes"], r["absmax_q"], r["absmax_s2"], w.size, 2)
    assert np.all(wp[:64 * 256] == 0)
    assert wp[64 * 256 + 5] == np.float32(fp8.decode(r["absmax_q"][256:257], fp8.E4M3)[0] *
                                          r["absmax_s2"][1] * np.float32(1.0))
