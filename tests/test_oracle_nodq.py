"""Pins for the oracle's store without double quantization (CPU only).

  * the pages' worked example (tests/golden/worked_example.json): a block of
    four values, its constant and three printed dequantized values;
  * an exact rational recomputation of single elements, w' = fl32(L[q] c);
  * the half-gap error bound (no second-level term);
  * agreement with the double-quantized values wherever c' = c (a block that
    holds its group's maximum) and disagreement elsewhere (the two stores
    are told apart);
  * the storage closed form: 4 + 32/64 = 4.5 bits per weight.
"""

import json
import os
from fractions import Fraction

import numpy as np

import oracle
from oracle import nf4
from oracle.bf16 import bf16_round


def _bf16(x):
    return bf16_round(np.asarray(x, dtype=np.float32))


def _fl32(x):
    """Correctly rounded float32 of a rational (nearest, ties to even)."""
    f = np.float32(float(x))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    return min(cands, key=lambda c: (abs(Fraction(float(c)) - x),
                                     int(np.float32(c).view(np.uint32)) & 1))


def test_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "worked_example.json")))
    block = _bf16(g["block"])
    st = oracle.quantize(block)
    assert st["absmax"][0] == np.max(np.abs(block))
    wp = oracle.dequantize_nodq(st["codes"], st["absmax"], 4)
    printed = np.array(g["dequantized_printed_approx"])
    for i in g["checked_dequantized_indices"]:
        assert abs(round(float(wp[i]), g["printed_decimals"]) - printed[i]) < 1e-9
    assert wp[3] == st["absmax"][0]  # level 1.0 times c


def test_elementwise_definition():
    rng = np.random.default_rng(4)
    w = _bf16(rng.standard_normal(64 * 500) * 0.02)
    st = oracle.quantize(w)
    wp = oracle.dequantize_nodq(st["codes"], st["absmax"], w.size)
    levels = oracle.codebook()
    for i in rng.integers(0, w.size, 300):
        c = st["absmax"][i // 64]
        want = _fl32(Fraction(float(levels[st["q"][i]])) * Fraction(float(c)))
        assert wp[i] == want


def test_error_bound_and_ragged_tail():
    rng = np.random.default_rng(5)
    for n in (1, 63, 64, 65, 64 * 257 + 5):
        w = _bf16(rng.standard_t(5, n) * 0.02)
        st = oracle.quantize(w)
        wp = oracle.dequantize_nodq(st["codes"], st["absmax"], n).astype(np.float64)
        levels = oracle.codebook().astype(np.float64)
        q = st["q"].astype(np.int64)
        gaps = np.diff(levels)
        half = np.maximum(np.concatenate([[gaps[0]], gaps])[q], np.concatenate([gaps, [gaps[-1]]])[q]) / 2
        c = st["absmax"][np.arange(n) // 64].astype(np.float64)
        assert np.all(np.abs(w.astype(np.float64) - wp) <= c * half + 1e-7 * c)
        assert st["absmax"].size == nf4.num_blocks(n)


def test_agrees_with_double_quant_where_constants_agree():
    rng = np.random.default_rng(6)
    w = _bf16(rng.standard_normal(16384 * 3) * 0.02)
    st = oracle.quantize(w)
    a = oracle.dequantize(st["codes"], st["absmax_q"], st["absmax_s2"], w.size)
    b = oracle.dequantize_nodq(st["codes"], st["absmax"], w.size)
    cprime = (oracle.level8()[st["absmax_q"]] * st["absmax_s2"][np.arange(st["absmax"].size) // 256]
              ).astype(np.float32)
    same = cprime == st["absmax"]
    assert same.sum() >= 3   # at least each group's maximum block
    blk = np.arange(w.size) // 64
    assert np.array_equal(a[same[blk]].view(np.uint32), b[same[blk]].view(np.uint32))
    assert not np.array_equal(a[~same[blk]], b[~same[blk]])


def test_storage_closed_form():
    assert nf4.bits_per_param(double_quant=False) == Fraction(9, 2)
    n = 4096 * 4096
    assert nf4.store_bytes(n, double_quant=False) == n // 2 + 4 * (n // 64)
    assert nf4.store_bytes(n, double_quant=False) * 8 == n * Fraction(9, 2)
