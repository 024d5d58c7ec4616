"""Pins for the oracle's linear forward/backward and bf16 rounding (CPU only).

  * bf16 rounding against torch's own float32 -> bfloat16 conversion;
  * forward output and all three gradients against torch.autograd in
    float64 on the dense (dequantized, bf16-rounded) weight: a dropped term,
    a wrong sign, a transposed operand or a missing scale fails here;
  * central finite differences of a scalar loss at the smallest workload's
    shape;
  * exact special cases: B = 0, A = 0, s = 0 and W' = 0.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.bf16 import bf16_round, f32_to_bf16_bits


def _bf16(x):
    return bf16_round(np.asarray(x, dtype=np.float32))


def test_bf16_round_matches_torch_random():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), want)


def test_bf16_round_matches_torch_ties():
    hi = np.arange(0, 1 << 16, 97, dtype=np.uint32)
    lows = np.array([0x0000, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    bits = (hi[:, None] << 16 | lows[None, :]).ravel().astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 3e38)]
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), want)


def _problem(M, N, K, r, seed=0, wscale=0.02):
    rng = np.random.default_rng(seed)
    X = _bf16(rng.standard_normal((M, K)))
    W = _bf16(rng.standard_normal((N, K)) * wscale)
    A = _bf16(rng.standard_normal((K, r)) * 0.01)
    B = _bf16(rng.standard_normal((r, N)) * 0.01)
    dY = _bf16(rng.standard_normal((M, N)) * 1e-3)
    st = oracle.quantize(W.ravel())
    wp = oracle.dequantize(st["codes"], st["absmax_q"], st["absmax_s2"], N * K).reshape(N, K)
    return X, wp, A, B, dY


def _torch_reference(X, wp, A, B, dY, s):
    Wb = torch.from_numpy(bf16_round(wp).astype(np.float64))
    Xt = torch.from_numpy(X.astype(np.float64)).requires_grad_(True)
    At = torch.from_numpy(A.astype(np.float64)).requires_grad_(True)
    Bt = torch.from_numpy(B.astype(np.float64)).requires_grad_(True)
    lin = torch.nn.functional.linear(Xt, Wb)  # X W^T
    Y = lin + s * torch.nn.functional.linear(torch.nn.functional.linear(Xt, At.T), Bt.T)
    Y.backward(torch.from_numpy(dY.astype(np.float64)))
    return Y.detach().numpy(), Xt.grad.numpy(), At.grad.numpy(), Bt.grad.numpy()


@pytest.mark.parametrize("shape", [(16, 256, 256, 8), (5, 192, 128, 3), (1, 64, 320, 16)])
def test_linear_matches_autograd(shape):
    M, N, K, r = shape
    X, wp, A, B, dY = _problem(M, N, K, r, seed=M + N)
    s = 2.0
    Y, T = oracle.linear_fwd(X, wp, A, B, s)
    dX, dA, dB = oracle.linear_bwd(dY, X, wp, A, B, s)
    Yr, dXr, dAr, dBr = _torch_reference(X, wp, A, B, dY, s)
    for got, want in ((Y, Yr), (dX, dXr), (dA, dAr), (dB, dBr)):
        assert got.shape == want.shape
        assert np.allclose(got, want, rtol=1e-12, atol=1e-15)
    assert np.allclose(T, X.astype(np.float64) @ A.astype(np.float64))


def test_linear_finite_differences():
    M, N, K, r = 16, 256, 256, 8
    X, wp, A, B, dY = _problem(M, N, K, r, seed=1)
    s = 2.0
    dX, dA, dB = oracle.linear_bwd(dY, X, wp, A, B, s)
    dYd = dY.astype(np.float64)

    def loss(Xv, Av, Bv):
        # the forward is affine in each argument, so a central difference of
        # L = <dY, Y> is exact up to float64 rounding
        Yv, _ = oracle.linear_fwd(Xv, wp, Av, Bv, s)
        return float(np.sum(Yv * dYd))

    rng = np.random.default_rng(2)
    h = 0.5
    for name, arr, grad in (("X", X, dX), ("A", A, dA), ("B", B, dB)):
        for _ in range(4):
            idx = tuple(int(rng.integers(0, d)) for d in arr.shape)
            p = arr.copy(); p[idx] += h
            m = arr.copy(); m[idx] -= h
            args = {"X": X, "A": A, "B": B}
            ap = dict(args); ap[name] = p
            am = dict(args); am[name] = m
            fd = (loss(ap["X"], ap["A"], ap["B"]) - loss(am["X"], am["A"], am["B"])) / (2 * h)
            g = grad[idx]
            assert abs(fd - g) <= 1e-9 * max(1.0, abs(g)) + 1e-12, (name, idx, fd, g)


def test_special_cases_exact():
    M, N, K, r = 8, 128, 192, 4
    X, wp, A, B, dY = _problem(M, N, K, r, seed=3)
    Wb = bf16_round(wp).astype(np.float64)
    base = X.astype(np.float64) @ Wb.T
    # B = 0: no adapter output, no gradient for A
    Y, _ = oracle.linear_fwd(X, wp, A, np.zeros_like(B), 2.0)
    assert np.array_equal(Y, base)
    _, dA, _ = oracle.linear_bwd(dY, X, wp, A, np.zeros_like(B), 2.0)
    assert np.all(dA == 0)
    # A = 0: no gradient for B, and dX has no adapter term
    dX, _, dB = oracle.linear_bwd(dY, X, wp, np.zeros_like(A), B, 2.0)
    assert np.all(dB == 0)
    assert np.array_equal(dX, dY.astype(np.float64) @ Wb)
    # s = 0: the plain NF4 product
    Y, _ = oracle.linear_fwd(X, wp, A, B, 0.0)
    assert np.array_equal(Y, base)
    # W' = 0: only the adapter term
    Y, _ = oracle.linear_fwd(X, np.zeros_like(wp), A, B, 0.5)
    want = 0.5 * ((X.astype(np.float64) @ A.astype(np.float64)) @ B.astype(np.float64))
    assert np.allclose(Y, want, rtol=1e-13, atol=0)


# --- planted mistakes in a copy of the oracle's backward: each must fail ----

def _bwd_variants():
    def drop_adapter_term(dY, X, wp, A, B, s):
        dX, dA, dB = oracle.linear_bwd(dY, X, wp, A, B, s)
        Wb = bf16_round(wp).astype(np.float64)
        return dY.astype(np.float64) @ Wb, dA, dB

    def transposed_B(dY, X, wp, A, B, s):
        dX, dA, dB = oracle.linear_bwd(dY, X, wp, A, B, s)
        return dX, dA, -dB

    def missing_scale(dY, X, wp, A, B, s):
        dX, dA, dB = oracle.linear_bwd(dY, X, wp, A, B, s)
        return dX, dA / s, dB

    def fp32_weight_not_bf16(dY, X, wp, A, B, s):
        dX, dA, dB = oracle.linear_bwd(dY, X, wp, A, B, s)
        d = dY.astype(np.float64) @ (wp.astype(np.float64) - bf16_round(wp).astype(np.float64))
        return dX + d, dA, dB

    return [drop_adapter_term, transposed_B, missing_scale, fp32_weight_not_bf16]


@pytest.mark.parametrize("bad", _bwd_variants())
def test_planted_backward_mistakes_are_caught(bad):
    M, N, K, r = 16, 256, 256, 8
    X, wp, A, B, dY = _problem(M, N, K, r, seed=4)
    s = 2.0
    _, dXr, dAr, dBr = _torch_reference(X, wp, A, B, dY, s)
    dX, dA, dB = bad(dY, X, wp, A, B, s)
    ok = all(np.allclose(g, w, rtol=1e-12, atol=1e-15) for g, w in ((dX, dXr), (dA, dAr), (dB, dBr)))
    assert not ok
