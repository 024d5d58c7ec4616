"""Pins for the oracle's quantize / double-quantize / dequantize (CPU only).

Pins used, none of which re-types the oracle's own arithmetic:
  * the pages' worked example (tests/golden/worked_example.json);
  * the closed forms the pages state (tests/golden/closed_forms.json);
  * exact (rational) brute force of the nearest-level rule on tiny blocks
    and on every float32 value next to each decision point;
  * a per-block reference written as plain Python loops over tiny tensors,
    including a ragged final block and group;
  * double-quantization invariants (q8 = 255 at the group maximum, half-step
    error bound) and the dequantization error bound.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import nf4
from oracle.bf16 import bf16_round


def _bf16(x):
    return bf16_round(np.asarray(x, dtype=np.float32))


# ----------------------------------------------------------------------------
# worked example
# ----------------------------------------------------------------------------

def test_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "worked_example.json")))
    block = _bf16(g["block"])
    c = np.max(np.abs(block))
    assert abs(float(c) - g["absmax_printed"]) < 5e-3  # bf16 of 0.80
    n = (block / c).astype(np.float32)
    assert np.array_equal(n, np.array(g["normalized_printed"], np.float32))
    st = oracle.quantize(block)
    # nearest NF4 levels of 0.125, -0.5, 0.0625, 1.0
    assert st["q"].tolist() == [9, 2, 8, 15]
    lv = oracle.codebook()[st["q"]]
    # the hypothetical levels agree with the real ones to two decimals
    # except for the first (0.1 vs 0.1609), which the page only supposed
    hyp = np.array(g["hypothetical_levels_printed"])
    assert np.all(np.abs(lv[1:] - hyp[1:]) < 0.006)
    assert lv[3] == 1.0
    # dequantized values: a 4-element tensor is one block and one group, so
    # c' = s2 = c exactly and w' = level * c
    wp = oracle.dequantize(st["codes"], st["absmax_q"], st["absmax_s2"], 4)
    printed = np.array(g["dequantized_printed_approx"])
    for i in g["checked_dequantized_indices"]:
        assert abs(round(float(wp[i]), g["printed_decimals"]) - printed[i]) < 1e-9
    assert st["absmax_q"].tolist() == [255]
    assert st["absmax_s2"][0] == c


# ----------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------

def _stack_params(shape):
    return shape["layers"] * sum(n * k for n, k in shape["linears"])


def _stack_bytes(shape):
    return shape["layers"] * sum(nf4.store_bytes(n * k) for n, k in shape["linears"])


def test_closed_forms(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "closed_forms.json")))
    no_dq = nf4.bits_per_param(double_quant=False)
    dq = nf4.bits_per_param()
    assert no_dq - 4 == Fraction(g["no_dq_overhead_bits_printed"]).limit_denominator()
    saving = no_dq - dq
    assert saving == Fraction(373046875, 10 ** 9)
    assert round(float(saving), g["dq_saving_bits_printed_decimals"]) == g["dq_saving_bits_printed"]
    assert dq == Fraction(4126953125, 10 ** 9)
    # block 64 is the only power of two whose saving rounds to 0.37
    for blk in (32, 128, 256):
        s = nf4.bits_per_param(block=blk, double_quant=False) - nf4.bits_per_param(block=blk)
        assert round(float(s), 2) != 0.37
    # the 65B-shaped stack: about 130 GB at 16 bits and about 33 GB stored
    sh = g["stack_65b_shape"]
    params = _stack_params(sh)
    assert params == 64_760_053_760
    assert round(2 * params / 1e9) == g["memory_65b_gb_16bit_printed"]
    b = _stack_bytes(sh)
    assert b == 33_407_713_280
    assert round(b / 1e9) == g["memory_65b_gb_4bit_printed"]
    # the 7B-shaped stack: about 14 GB at 16 bits, 3.5 GB plus a small overhead
    sh7 = g["stack_7b_shape"]
    p7 = _stack_params(sh7)
    assert round(2 * p7 / 1e9) in (13, 14)  # linears only; embeddings excluded
    b7 = _stack_bytes(sh7)
    assert b7 == 3_340_771_328
    assert 0 < b7 - p7 / 2 < 0.05 * p7 / 2  # "plus small overhead"
    # single stores used by the workloads
    assert nf4.store_bytes(4096 * 4096) == 8_654_848
    assert nf4.store_bytes(256 * 256) == 33_808


# ----------------------------------------------------------------------------
# nearest-level rule, exact
# ----------------------------------------------------------------------------

def _exact_nearest(nval, levels):
    """Rational brute force: index of the nearest level, ties to the lower."""
    x = Fraction(float(nval))
    best, bestd = None, None
    for j, l in enumerate(levels):
        d = abs(x - Fraction(float(l)))
        if bestd is None or d < bestd:
            best, bestd = j, d
    return best


def test_nearest_level_at_every_decision_point():
    levels = oracle.codebook()
    vals = []
    for j in range(15):
        mid = (float(levels[j]) + float(levels[j + 1])) / 2.0
        f = np.float32(mid)
        for _ in range(4):
            f = np.nextafter(f, np.float32(-2))
        for _ in range(9):
            vals.append(f)
            f = np.nextafter(f, np.float32(2))
    vals += [np.float32(v) for v in (-1.0, 1.0, 0.0, -0.0, 1e-30, -1e-30, 1e-45)]
    vals = np.array(vals, dtype=np.float32)
    got = oracle.nearest_level(vals)
    for v, q in zip(vals, got):
        assert q == _exact_nearest(v, levels), v


def test_nearest_level_random_exact():
    rng = np.random.default_rng(1)
    levels = oracle.codebook()
    vals = rng.uniform(-1, 1, 3000).astype(np.float32)
    got = oracle.nearest_level(vals)
    for v, q in zip(vals, got):
        assert q == _exact_nearest(v, levels)


# ----------------------------------------------------------------------------
# plain-loop reference for tiny tensors (blocking, packing, groups)
# ----------------------------------------------------------------------------

def _loop_reference(w, block, group):
    levels = oracle.codebook()
    w = [np.float32(x) for x in w]
    n = len(w)
    q, absmax = [], []
    for b0 in range(0, n, block):
        blk = w[b0:b0 + block]
        c = np.float32(max(abs(x) for x in blk))
        absmax.append(c)
        for x in blk:
            nn = np.float32(0.0) if c == 0 else np.float32(x / c)
            q.append(_exact_nearest(nn, levels))
    q8, s2 = [], []
    for g0 in range(0, len(absmax), group):
        grp = absmax[g0:g0 + group]
        m = np.float32(max(grp))
        s2.append(m)
        for c in grp:
            if m == 0:
                q8.append(0)
            else:
                r = np.float32(np.float32(c / m) * np.float32(255.0))
                q8.append(int(np.rint(r)))
    packed = []
    for i in range(0, n, 2):
        lo = q[i]
        hi = q[i + 1] if i + 1 < n else 0
        packed.append(lo | (hi << 4))
    return q, packed, q8, s2, absmax


@pytest.mark.parametrize("numel", [1, 2, 3, 63, 64, 65, 127, 200, 64 * 256 + 77, 64 * 512 + 1])
def test_quantize_matches_loop_reference(numel):
    rng = np.random.default_rng(numel)
    w = _bf16(rng.standard_normal(numel) * 0.02)
    # plant structure: an all-zero block, a lone non-zero, a negative absmax
    if numel > 200:
        w[64:128] = 0
        w[128:192] = 0
        w[130] = np.float32(-0.5)
        w[256:320] *= 1000  # an outlier block inside the first group
    st = oracle.quantize(w)
    q, packed, q8, s2, absmax = _loop_reference(w, nf4.BLOCK, nf4.GROUP)
    assert st["q"].tolist() == q
    assert st["codes"].tolist() == packed
    assert st["absmax_q"].tolist() == q8
    assert np.array_equal(st["absmax_s2"], np.array(s2, np.float32))
    assert np.array_equal(st["absmax"], np.array(absmax, np.float32))


def test_tiny_blocks_brute_force():
    """Blocksizes 4 and 8 with the loop reference: exercises the blocking
    independently of the production block size."""
    rng = np.random.default_rng(7)
    for block in (4, 8):
        w = _bf16(rng.standard_normal(40))
        q, packed, q8, s2, absmax = _loop_reference(w, block, 3)
        levels = oracle.codebook()
        # dequant(quant(x)) is the nearest representable value in each block
        for i, x in enumerate(w):
            c = absmax[i // block]
            cand = [abs(Fraction(float(x)) - Fraction(float(l)) * Fraction(float(c))) for l in levels]
            # nearest in the normalized domain equals nearest in the scaled one
            # up to the float32 rounding of x/c; check it is optimal or a tie
            best = min(cand)
            chosen = cand[q[i]]
            assert chosen - best <= Fraction(float(c)) * Fraction(1, 2 ** 23)


def test_pack_unpack_roundtrip():
    rng = np.random.default_rng(3)
    for n in (1, 2, 7, 64, 1001):
        q = rng.integers(0, 16, n).astype(np.uint8)
        p = oracle.pack_codes(q)
        assert p.size == (n + 1) // 2
        assert np.array_equal(oracle.unpack_codes(p, n), q)
        if n % 2:
            assert p[-1] >> 4 == 0


def test_all_zero_tensor():
    st = oracle.quantize(np.zeros(64 * 300, np.float32))
    assert np.all(st["q"] == 7)
    assert np.all(st["absmax_q"] == 0)
    assert np.all(st["absmax_s2"] == 0)
    wp = oracle.dequantize(st["codes"], st["absmax_q"], st["absmax_s2"], 64 * 300)
    assert np.all(wp == 0)


def test_level_endpoints_hit_by_absmax_element():
    rng = np.random.default_rng(11)
    w = _bf16(rng.standard_normal(64 * 64))
    st = oracle.quantize(w)
    q = st["q"].reshape(-1, 64)
    wb = w.reshape(-1, 64)
    for b in range(q.shape[0]):
        i = int(np.argmax(np.abs(wb[b])))
        assert q[b, i] == (15 if wb[b, i] > 0 else 0)


# ----------------------------------------------------------------------------
# double quantization and dequantization bounds
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("dist", ["normal", "student_t"])
def test_double_quant_invariants_and_error_bound(dist):
    rng = np.random.default_rng(5)
    n = 64 * 256 * 6 + 64 * 37
    if dist == "normal":
        w = _bf16(rng.standard_normal(n) * 0.02)
    else:
        w = _bf16(rng.standard_t(5.0, n) * 0.02)
    st = oracle.quantize(w)
    c = st["absmax"]
    q8 = st["absmax_q"].astype(np.int64)
    s2 = st["absmax_s2"]
    g = np.arange(c.size) // nf4.GROUP
    # the group maximum is coded 255
    for gi in range(s2.size):
        sel = np.where(g == gi)[0]
        assert q8[sel[np.argmax(c[sel])]] == 255
        assert s2[gi] == c[sel].max()
    # q8 is the nearest integer to 255 c / s2 (exact rational), up to the
    # float32 rounding of the ratio
    for b in range(0, c.size, 7):
        r = 255 * Fraction(float(c[b])) / Fraction(float(s2[g[b]]))
        assert abs(Fraction(int(q8[b])) - r) <= Fraction(1, 2) + Fraction(1, 10 ** 4)
    l8 = oracle.level8()
    cp = (l8[q8] * s2[g]).astype(np.float64)
    # half-step bound of a linear 8-bit code, plus float32 rounding slack
    bound = s2[g].astype(np.float64) / 510.0 + 4 * np.spacing(s2[g]).astype(np.float64)
    assert np.all(np.abs(cp - c) <= bound)
    assert np.all(cp[q8 == 255] == s2[g][q8 == 255])
    # dequantization error bound per element
    wp = oracle.dequantize(st["codes"], st["absmax_q"], st["absmax_s2"], n).astype(np.float64)
    levels = oracle.codebook().astype(np.float64)
    qq = st["q"].astype(np.int64)
    gaps = np.diff(levels)
    half_gap = np.maximum(np.concatenate([[gaps[0]], gaps])[qq], np.concatenate([gaps, [gaps[-1]]])[qq]) / 2
    blk = np.arange(n) // nf4.BLOCK
    err = np.abs(w.astype(np.float64) - wp)
    lim = c[blk] * half_gap + np.abs(levels[qq]) * np.abs(c[blk] - cp[blk]) + 1e-7 * c[blk]
    assert np.all(err <= lim)


def _fl32(x):
    """Correctly rounded float32 of a rational (nearest, ties to even)."""
    f = np.float32(float(x))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = min(cands, key=lambda c: (abs(Fraction(float(c)) - x), int(np.float32(c).view(np.uint32)) & 1))
    return np.float32(best)


def test_dequantize_elementwise_definition():
    """Two roundings in order (never fused): spot-check against Fractions."""
    rng = np.random.default_rng(9)
    w = _bf16(rng.standard_normal(64 * 300) * 0.02)
    st = oracle.quantize(w)
    wp = oracle.dequantize(st["codes"], st["absmax_q"], st["absmax_s2"], w.size)
    levels = oracle.codebook()
    for i in rng.integers(0, w.size, 200):
        b = i // 64
        gi = b // 256
        l8 = _fl32(Fraction(int(st["absmax_q"][b]), 255))
        cprime = np.float32(Fraction(float(l8)) * Fraction(float(st["absmax_s2"][gi])))
        want = np.float32(Fraction(float(levels[st["q"][i]])) * Fraction(float(cprime)))
        assert wp[i] == want
