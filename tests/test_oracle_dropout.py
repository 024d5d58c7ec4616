"""Pins for the oracle's LoRA dropout (CPU only).

  * Philox4x32-10 against the generator's published known-answer vectors;
  * the keep mask: p = 0 keeps everything, the dropped fraction at p = 0.05
    lies within six binomial standard deviations of thr / 2^16, seeds and
    offsets give different masks, the mask depends only on the flat element
    index (leading rows of a taller input), the threshold's rounding;
  * the linear layer with a fixed mask against torch.autograd in float64
    (nn.functional.dropout's own formula with that mask: the kept elements
    scaled by the inverse keep probability), and an all-ones mask with
    scale 1 against the plain layer;
  * a planted mistake (the input gradient's adapter term left unmasked) fails.
"""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.bf16 import bf16_round


def test_philox_known_answers(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "philox_kat.json")))
    for vec in g["vectors"]:
        ctr = np.array([int(x, 16) for x in vec["counter"]], dtype=np.uint32)
        key = [int(x, 16) for x in vec["key"]]
        out = oracle.philox4x32_10(ctr, key)
        assert [int(v) for v in out] == [int(x, 16) for x in vec["output"]]


def test_philox_vectorized_equals_single():
    rng = np.random.default_rng(0)
    ctr = rng.integers(0, 1 << 32, size=(50, 4), dtype=np.uint64).astype(np.uint32)
    many = oracle.philox4x32_10(ctr, (123, 456))
    for i in range(50):
        assert np.array_equal(many[i], oracle.philox4x32_10(ctr[i], (123, 456)))


def test_threshold_rounding():
    assert oracle.keep_threshold(0.0) == 0
    assert oracle.keep_threshold(0.05) == 3277       # 3276.8 -> 3277
    assert oracle.keep_threshold(0.5) == 32768
    assert oracle.keep_threshold(0.1) == 6554         # 6553.6 -> 6554
    assert oracle.keep_scale(0.5) == 2.0
    with pytest.raises(ValueError):
        oracle.keep_threshold(1.0)
    with pytest.raises(ValueError):
        oracle.keep_threshold(-0.1)


def test_keep_all_at_zero():
    keep = oracle.dropout_keep(64, 256, 0.0, seed=5)
    assert keep.all()


def test_drop_fraction_binomial():
    M, K = 2048, 2048
    keep = oracle.dropout_keep(M, K, 0.05, seed=1234, offset=7)
    n = M * K
    q = oracle.keep_threshold(0.05) / 65536.0
    dropped = n - int(keep.sum())
    sd = np.sqrt(n * q * (1 - q))
    assert abs(dropped - n * q) < 6 * sd
    # no visible structure along rows or columns
    rows = (~keep).sum(axis=1)
    cols = (~keep).sum(axis=0)
    assert abs(rows.mean() - K * q) < 6 * np.sqrt(K * q * (1 - q) / M)
    assert abs(cols.mean() - M * q) < 6 * np.sqrt(M * q * (1 - q) / K)
    # the 16-bit halves of one generator call are not tied together
    pairs = (~keep).reshape(-1, 2)
    both = int(np.sum(pairs[:, 0] & pairs[:, 1]))
    assert abs(both - pairs.shape[0] * q * q) < 6 * np.sqrt(pairs.shape[0] * q * q)


def test_seed_offset_and_prefix():
    a = oracle.dropout_keep(128, 512, 0.3, seed=1, offset=0)
    b = oracle.dropout_keep(128, 512, 0.3, seed=2, offset=0)
    c = oracle.dropout_keep(128, 512, 0.3, seed=1, offset=1)
    d = oracle.dropout_keep(128, 512, 0.3, seed=1 << 40, offset=0)
    assert not np.array_equal(a, b) and not np.array_equal(a, c) and not np.array_equal(a, d)
    tall = oracle.dropout_keep(300, 512, 0.3, seed=1, offset=0)
    assert np.array_equal(tall[:128], a)


def test_pack_roundtrip():
    keep = oracle.dropout_keep(16, 320, 0.4, seed=9)
    words = oracle.pack_keep(keep)
    assert words.shape == (16, 10) and words.dtype == np.uint32
    assert np.array_equal(oracle.unpack_keep(words, 320), keep)
    # bit j of word w is element 32 w + j
    assert bool(words[3, 2] >> 5 & 1) == bool(keep[3, 69])


def _problem(M, N, K, r, seed):
    rng = np.random.default_rng(seed)
    X = bf16_round(rng.standard_normal((M, K)).astype(np.float32))
    W = bf16_round((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    A = bf16_round((rng.standard_normal((K, r)) * 0.05).astype(np.float32))
    B = bf16_round((rng.standard_normal((r, N)) * 0.05).astype(np.float32))
    dY = bf16_round((rng.standard_normal((M, N)) * 1e-2).astype(np.float32))
    st = oracle.quantize(W.ravel())
    wp = oracle.dequantize(st["codes"], st["absmax_q"], st["absmax_s2"], N * K).reshape(N, K)
    return X, wp, A, B, dY


def _torch_dropout_reference(X, wp, A, B, dY, s, keep, p_real):
    Wb = torch.from_numpy(bf16_round(wp).astype(np.float64))
    Xt = torch.from_numpy(X.astype(np.float64)).requires_grad_(True)
    At = torch.from_numpy(A.astype(np.float64)).requires_grad_(True)
    Bt = torch.from_numpy(B.astype(np.float64)).requires_grad_(True)
    mask = torch.from_numpy(keep.astype(np.float64))
    Xd = Xt * mask / (1.0 - p_real)   # inverted dropout with this mask
    T = Xd @ At
    Y = Xt @ Wb.T + s * (T @ Bt)
    Y.backward(torch.from_numpy(dY.astype(np.float64)))
    return Y.detach().numpy(), T.detach().numpy(), Xt.grad.numpy(), At.grad.numpy(), Bt.grad.numpy()


@pytest.mark.parametrize("shape,p", [((16, 128, 256, 8), 0.05), ((7, 64, 192, 3), 0.5),
                                     ((32, 192, 128, 64), 0.1)])
def test_dropout_linear_matches_autograd(shape, p):
    M, N, K, r = shape
    X, wp, A, B, dY = _problem(M, N, K, r, seed=M + K)
    keep = oracle.dropout_keep(M, K, p, seed=77, offset=3)
    ks = oracle.keep_scale(p)
    p_real = oracle.keep_threshold(p) / 65536.0
    s = 0.25
    Y, T = oracle.linear_fwd(X, wp, A, B, s, keep=keep, keep_scale=ks)
    dX, dA, dB = oracle.linear_bwd(dY, X, wp, A, B, s, keep=keep, keep_scale=ks)
    Yr, Tr, dXr, dAr, dBr = _torch_dropout_reference(X, wp, A, B, dY, s, keep, p_real)
    for got, want in ((Y, Yr), (T, Tr), (dX, dXr), (dA, dAr), (dB, dBr)):
        assert np.allclose(got, want, rtol=1e-12, atol=1e-14)


def test_all_ones_mask_is_plain_layer():
    M, N, K, r = 8, 128, 192, 4
    X, wp, A, B, dY = _problem(M, N, K, r, seed=3)
    keep = np.ones((M, K), bool)
    Y0, T0 = oracle.linear_fwd(X, wp, A, B, 2.0)
    Y1, T1 = oracle.linear_fwd(X, wp, A, B, 2.0, keep=keep, keep_scale=1.0)
    assert np.array_equal(Y0, Y1) and np.array_equal(T0, T1)
    g0 = oracle.linear_bwd(dY, X, wp, A, B, 2.0)
    g1 = oracle.linear_bwd(dY, X, wp, A, B, 2.0, keep=keep, keep_scale=1.0)
    for a, b in zip(g0, g1):
        assert np.array_equal(a, b)


def test_planted_unmasked_input_gradient_is_caught():
    M, N, K, r = 16, 128, 256, 8
    X, wp, A, B, dY = _problem(M, N, K, r, seed=11)
    p = 0.3
    keep = oracle.dropout_keep(M, K, p, seed=1)
    ks = oracle.keep_scale(p)
    s = 0.5
    _, _, dXr, _, _ = _torch_dropout_reference(X, wp, A, B, dY, s, keep, oracle.keep_threshold(p) / 65536.0)
    # mistake: the adapter's input-gradient term without the mask
    dX, _, _ = oracle.linear_bwd(dY, X, wp, A, B, s)
    Wb = bf16_round(wp).astype(np.float64)
    lr = dX - dY.astype(np.float64) @ Wb
    bad = dY.astype(np.float64) @ Wb + lr * ks
    assert not np.allclose(bad, dXr, rtol=1e-9, atol=1e-12)
