"""GPU parity of the NF4 store without double quantization (one float32
constant per 64-block) against the oracle.

  * quantization bit for bit: codes (the same as the double-quantized
    store's) and the float32 block constants, on workload weight shapes,
    ragged sizes and special blocks;
  * dequantization bit for bit (float32 and bf16 out);
  * the compute weight inside the fused kernels bit for bit: one-hot token
    rows and a zero adapter make every output a single bf16(w') (GEMV for
    M <= 16, the MFMA forward and dX otherwise) -- the constants of the two
    stores differ by under one percent, which the linear tolerance alone
    would not see;
  * forward and backward within the linear tolerance on both paths, and the
    adapter merge bit for bit.
"""

import numpy as np
import pytest
import torch

import oracle
import synthetic
from tests.gpu_util import assert_close, device, host_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    device()
    import bit_quantized_finetuning_quantize_amd as q
    return q


def _oracle_nodq(w):
    ref = oracle.quantize(host_f32(w).ravel())
    wp = oracle.dequantize_nodq(ref["codes"], ref["absmax"], ref["numel"])
    return ref, wp


def _check_store(q, w, label):
    print(f"[case] nodq store {label} numel={w.numel()}", flush=True)
    st = q.qlora_nf4_quantize(w, double_quant=False)
    assert st.absmax_q is None and not st.double_quant
    wp32 = q.qlora_nf4_dequantize(st)
    wp16 = q.qlora_nf4_dequantize_bf16(st)
    torch.cuda.synchronize()
    ref, wp = _oracle_nodq(w)
    assert np.array_equal(st.codes.cpu().numpy(), ref["codes"]), label + " codes"
    c = st.absmax_s2.cpu().numpy()
    assert c.shape == ref["absmax"].shape
    assert np.array_equal(c.view(np.uint32), ref["absmax"].view(np.uint32)), label + " constants"
    assert np.array_equal(wp32.cpu().numpy().view(np.uint32), wp.view(np.uint32)), label + " f32"
    got16 = wp16.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got16, oracle.f32_to_bf16_bits(wp)), label + " bf16"
    return st, ref, wp


def test_workload_weights(q):
    dev = device()
    for (N, K), seed in (((256, 256), 0), ((4096, 4096), 1), ((11008, 4096), 2)):
        w = synthetic.normal((N, K), 0.02, dev, seed, synthetic.W_IDX)
        _check_store(q, w, f"W {N}x{K}")


@pytest.mark.parametrize("numel", [1, 63, 64, 65, 16385, 64 * 256 * 3 + 17])
def test_ragged_sizes(q, numel):
    w = synthetic.normal((numel,), 0.02, device(), 4, numel)
    _check_store(q, w, f"ragged {numel}")


def test_special_blocks(q):
    dev = device()
    rng = np.random.default_rng(1)
    v = (rng.standard_normal(16384 * 2) * 0.02).astype(np.float32)
    v[0:64] = 0
    v[64 * 3:64 * 4] *= 1e4
    v[64 * 5:64 * 6] = np.float32(1e-39)
    v[64 * 7 + 3] = -5.0
    w = torch.from_numpy(v).to(torch.bfloat16).to(dev)
    _check_store(q, w, "special blocks")


def test_codes_same_as_double_quant(q):
    w = synthetic.student_t((2048, 4096), 5, 0.02, device(), 0, synthetic.W_IDX)
    a = q.qlora_nf4_quantize(w)
    b = q.qlora_nf4_quantize(w, double_quant=False)
    torch.cuda.synchronize()
    assert torch.equal(a.codes, b.codes)
    assert b.nbytes() * 8 == w.numel() * 4.5


@pytest.mark.parametrize("M,N,K", [(1, 256, 512), (16, 384, 320), (64, 384, 320),
                                   (160, 192, 640)])
def test_compute_weight_bit_exact(q, M, N, K):
    dev = device()
    print(f"[case] nodq one-hot compute weight M={M} N={N} K={K}", flush=True)
    r = 8
    W, _, _, _, _ = synthetic.linear_inputs(M, N, K, r, dev, seed=7, need_dy=False)
    st = q.qlora_nf4_quantize(W, double_quant=False)
    _, wp = _oracle_nodq(W)
    wpb = oracle.bf16_round(wp.reshape(N, K))
    rng = np.random.default_rng(M * 7 + N + K)
    ks = rng.integers(0, K, size=M)
    X = torch.zeros(M, K, dtype=torch.bfloat16, device=dev)
    X[torch.arange(M), torch.as_tensor(ks, device=dev)] = 1.0
    A = torch.zeros(K, r, dtype=torch.bfloat16, device=dev)
    B = torch.zeros(r, N, dtype=torch.bfloat16, device=dev)
    Y, T = q.qlora_linear_fwd(X, st, A, B, 2.0)
    ns = rng.integers(0, N, size=M)
    dY = torch.zeros(M, N, dtype=torch.bfloat16, device=dev)
    dY[torch.arange(M), torch.as_tensor(ns, device=dev)] = 1.0
    dX, _, _ = q.qlora_linear_bwd(dY, X, T, st, A, B, 2.0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_f32(Y), wpb[:, ks].T.astype(np.float32),
                                  err_msg="forward weights")
    np.testing.assert_array_equal(host_f32(dX), wpb[ns, :].astype(np.float32),
                                  err_msg="dX weights")


@pytest.mark.parametrize("shape", [(4, 4096, 4096, 16), (300, 320, 192, 16),
                                   (513, 384, 448, 100)])
def test_linear_parity(q, shape):
    M, N, K, r = shape
    dev = device()
    print(f"[case] nodq linear M={M} N={N} K={K} r={r}", flush=True)
    W, X, A, B, dY = synthetic.linear_inputs(M, N, K, r, dev, seed=M + K)
    s = 2.0
    st = q.qlora_nf4_quantize(W, double_quant=False)
    Y, T = q.qlora_linear_fwd(X, st, A, B, s)
    dX, dA, dB = q.qlora_linear_bwd(dY, X, T, st, A, B, s)
    torch.cuda.synchronize()
    _, wp = _oracle_nodq(W)
    wp = wp.reshape(N, K)
    Xh, Ah, Bh, dYh = host_f32(X), host_f32(A), host_f32(B), host_f32(dY)
    Yo, To = oracle.linear_fwd(Xh, wp, Ah, Bh, s)
    dXo, dAo, dBo = oracle.linear_bwd(dYh, Xh, wp, Ah, Bh, s)
    assert_close(host_f32(Y), Yo, "nodq Y")
    assert_close(host_f32(T), To, "nodq T", tol=1e-5)
    assert_close(host_f32(dX), dXo, "nodq dX")
    assert_close(host_f32(dA), dAo, "nodq dA")
    assert_close(host_f32(dB), dBo, "nodq dB")


def test_merge_bit_exact(q):
    dev = device()
    N, K, r, s = 192, 256, 40, 0.37
    print(f"[case] nodq merge N={N} K={K} r={r}", flush=True)
    W, _, A, B, _ = synthetic.linear_inputs(8, N, K, r, dev, seed=12, need_dy=False)
    A = (A.float() * 30).to(torch.bfloat16)
    B = (B.float() * 30).to(torch.bfloat16)
    st = q.qlora_nf4_quantize(W, double_quant=False)
    out = q.qlora_nf4_merge(st, A, B, s)
    torch.cuda.synchronize()
    _, wp = _oracle_nodq(W)
    want = oracle.merge(wp.reshape(N, K), host_f32(A), host_f32(B), s)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want)
