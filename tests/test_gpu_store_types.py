"""GPU parity for the store types beside NF4 with the linear constant code:
FP4 levels (QLORA_STORE_FP4), the E4M3 code for the block constants
(QLORA_STORE_DQ_FP8), both, and FP4 without double quantization. Against
oracle.store: codes, 8-bit constants and second-level constants bit for bit,
float32 and bf16 dequantization bit for bit, the compute weight bf16(w')
inside the GEMV, MFMA forward and input-gradient kernels bit for bit
(one-hot token rows), forward and backward within the linear tolerance on
both paths, and the adapter merge bit for bit."""

import numpy as np
import pytest
import torch

import oracle
import synthetic
from oracle import store as ostore
from oracle.bf16 import bf16_round, f32_to_bf16_bits
from tests.gpu_util import assert_close, device, host_f32

pytestmark = pytest.mark.gpu

TYPES = [1, 2, 3]


@pytest.fixture(scope="module")
def q():
    device()
    import bit_quantized_finetuning_quantize_amd as q
    return q


def _ref(w, st_type, dq=True):
    return ostore.quantize(host_f32(w).ravel(), st_type, double_quant=dq)


def _check_store(st, ref, label):
    torch.cuda.synchronize()
    assert np.array_equal(st.codes.cpu().numpy(), ref["codes"]), f"{label}: codes"
    if ref["absmax_q"] is not None:
        assert np.array_equal(st.absmax_q.cpu().numpy(), ref["absmax_q"]), f"{label}: absmax_q"
    assert np.array_equal(st.absmax_s2.cpu().numpy().view(np.uint32),
                          ref["absmax_s2"].view(np.uint32)), f"{label}: absmax_s2"


def _roundtrip(q, w, st_type, label, dq=True):
    print(f"[case] {label} type={st_type} dq={dq} numel={w.numel()}", flush=True)
    st = q.qlora_nf4_quantize(w, double_quant=dq, store_type=st_type)
    ref = _ref(w, st_type, dq)
    _check_store(st, ref, label)
    wp = q.qlora_nf4_dequantize(st)
    wpb = q.qlora_nf4_dequantize_bf16(st)
    torch.cuda.synchronize()
    want = ostore.dequantize(ref["codes"], ref["absmax_q"], ref["absmax_s2"], w.numel(), st_type)
    assert np.array_equal(wp.cpu().numpy().view(np.uint32), want.view(np.uint32)), \
        f"{label}: fp32 dequant"
    gotb = wpb.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(gotb, f32_to_bf16_bits(want)), f"{label}: bf16 dequant"
    return st, ref, want


@pytest.mark.parametrize("st_type", TYPES)
def test_workload_and_student_t_weights(q, st_type):
    dev = device()
    for label, w in (("4096x4096 N(0,0.02)", synthetic.normal((4096, 4096), 0.02, dev, 0, 0)),
                     ("11008x4096 t5", synthetic.student_t((11008, 4096), 5, 0.02, dev, 0, 1)),
                     ("ragged 16384*3+77", synthetic.normal((16384 * 3 + 77,), 0.02, dev, 2, 0))):
        _roundtrip(q, w, st_type, label)


def test_fp4_without_double_quantization(q):
    dev = device()
    w = synthetic.student_t((1000, 192), 5, 0.02, dev, 4, 0)
    _roundtrip(q, w, 1, "fp4 no-dq", dq=False)
    # the constant-code flag has no effect without double quantization
    _roundtrip(q, w, 3, "fp4 no-dq, flag 2 set", dq=False)


def _grid_blocks(cs):
    """Blocks whose absmax is c, filled with every bf16 value of [-c, c]."""
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    vals = (bits << 16).view(np.float32)
    out = []
    for c in cs:
        cb = float(bf16_round(np.float32(c)))
        sel = vals[np.isfinite(vals) & (np.abs(vals) <= cb)]
        nb = -(-sel.size // 63)
        blocks = np.zeros((nb, 64), np.float32)
        blocks[:, 0] = cb
        blocks[1::2, 0] = -cb
        blocks[:, 1:] = np.concatenate([sel, np.zeros(nb * 63 - sel.size, np.float32)]).reshape(nb, 63)
        out.append(blocks.ravel())
    return np.concatenate(out)


def test_fp4_every_mantissa_pair(q):
    """Every bf16 mantissa of c in [1, 2) against every bf16 value of [-c, c]
    (every quotient the FP4 decision thresholds can see), with both constant
    codes, and c at the ends of the float32 range."""
    dev = device()
    cs = [1.0 + m / 128.0 for m in range(128)] + [2.0 ** -120, 2.0 ** 120]
    w = torch.from_numpy(_grid_blocks(cs)).to(torch.bfloat16).to(dev)
    _roundtrip(q, w, 1, "fp4 bf16 grid")
    _roundtrip(q, w, 3, "fp4+fp8 bf16 grid")


@pytest.mark.parametrize("st_type", TYPES)
def test_special_blocks(q, st_type):
    dev = device()
    rng = np.random.default_rng(0)
    n = 16384 * 3
    v = (rng.standard_normal(n) * 0.02).astype(np.float32)
    v[0:64] = 0
    v[16384:32768] = 0                 # all-zero group: S = 0
    v[64 * 5:64 * 6] = 0
    v[64 * 5 + 17] = -1e-3
    v[64 * 9:64 * 10] *= 1e4           # outlier block: the others far below 448 S
    v[64 * 11:64 * 12] = np.float32(1e-39)
    v[64 * 12:64 * 13] = -np.float32(2.0 ** -126)
    w = torch.from_numpy(v).to(torch.bfloat16).to(dev)
    _roundtrip(q, w, st_type, "special blocks")


@pytest.mark.parametrize("st_type", TYPES)
@pytest.mark.parametrize("M,N,K", [(16, 256, 512), (1, 192, 640), (64, 384, 320), (300, 192, 640)])
def test_compute_weight_bit_exact_in_products(q, st_type, M, N, K):
    """One-hot token rows and a zero adapter: Y[m][n] = bf16(w'[n][k_m]) and,
    with one-hot dY rows, dX = bf16(w'[n_m][k]), bit for bit, on the GEMV
    (M <= 16) and the MFMA forward and input-gradient kernels."""
    dev = device()
    print(f"[case] one-hot type={st_type} M={M} N={N} K={K}", flush=True)
    r = 8
    W = synthetic.student_t((N, K), 5, 0.02, dev, M + st_type, 0)
    st = q.qlora_nf4_quantize(W, store_type=st_type)
    ref = _ref(W, st_type)
    wp = ostore.dequantize(ref["codes"], ref["absmax_q"], ref["absmax_s2"], N * K,
                           st_type).reshape(N, K)
    wpb = bf16_round(wp)
    rng = np.random.default_rng(M + N + K + st_type)
    ks = rng.integers(0, K, size=M)
    X = torch.zeros(M, K, dtype=torch.bfloat16, device=dev)
    X[torch.arange(M), torch.as_tensor(ks, device=dev)] = 1.0
    A = torch.zeros(K, r, dtype=torch.bfloat16, device=dev)
    B = torch.zeros(r, N, dtype=torch.bfloat16, device=dev)
    Y, T = q.qlora_linear_fwd(X, st, A, B, 2.0)
    ns = rng.integers(0, N, size=M)
    dY = torch.zeros(M, N, dtype=torch.bfloat16, device=dev)
    dY[torch.arange(M), torch.as_tensor(ns, device=dev)] = 1.0
    dX, dA, dB = q.qlora_linear_bwd(dY, X, T, st, A, B, 2.0)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_f32(Y), wpb[:, ks].T.astype(np.float32),
                                  err_msg="forward weights")
    np.testing.assert_array_equal(host_f32(dX), wpb[ns, :].astype(np.float32),
                                  err_msg="dX weights")


@pytest.mark.parametrize("st_type", TYPES)
@pytest.mark.parametrize("shape", [(16, 256, 256, 8), (1, 4096, 4096, 16), (300, 384, 448, 100),
                                   (2048, 11008, 4096, 64)])
def test_linear_parity(q, st_type, shape):
    """Forward and backward within the bf16 tolerance on both paths, the
    workload-sized MLP projection included (sampled rows)."""
    M, N, K, r = shape
    dev = device()
    label = f"type={st_type} M={M} N={N} K={K} r={r}"
    print(f"[case] {label}", flush=True)
    W, X, A, B, dY = synthetic.linear_inputs(M, N, K, r, dev, seed=st_type + M,
                                             weight="student_t")
    s = 2.0 / r
    st = q.qlora_nf4_quantize(W, store_type=st_type)
    Y, T = q.qlora_linear_fwd(X, st, A, B, s)
    dX, dA, dB = q.qlora_linear_bwd(dY, X, T, st, A, B, s)
    torch.cuda.synchronize()
    ref = _ref(W, st_type)
    _check_store(st, ref, label)
    wp = ostore.dequantize(ref["codes"], ref["absmax_q"], ref["absmax_s2"], N * K,
                           st_type).reshape(N, K)
    rows = np.arange(M) if M <= 512 else np.sort(np.random.default_rng(1).choice(M, 64, False))
    Xh, Ah, Bh, dYh = host_f32(X), host_f32(A), host_f32(B), host_f32(dY)
    Yo, To = oracle.linear_fwd(Xh[rows], wp, Ah, Bh, s)
    assert_close(host_f32(Y)[rows], Yo, label + " Y")
    dXo, _, _ = oracle.linear_bwd(dYh[rows], Xh[rows], wp, Ah, Bh, s)
    assert_close(host_f32(dX)[rows], dXo, label + " dX")
    _, dAo, dBo = oracle.linear_bwd(dYh, Xh, np.zeros((N, K), np.float32), Ah, Bh, s)
    assert_close(host_f32(dA), dAo, label + " dA")
    assert_close(host_f32(dB), dBo, label + " dB")


@pytest.mark.parametrize("st_type", TYPES)
def test_merge_bit_exact(q, st_type):
    """bf16(w' + s (A B)^T) with the type's w' (the merge oracle applied to
    the type's dequantized weight, which it takes as an input)."""
    dev = device()
    N, K, r, s = 192, 320, 16, 0.5
    W, _, A, B, _ = synthetic.linear_inputs(8, N, K, r, dev, seed=st_type, need_dy=False,
                                            weight="student_t")
    st = q.qlora_nf4_quantize(W, store_type=st_type)
    out = q.qlora_nf4_merge(st, A, B, s)
    torch.cuda.synchronize()
    ref = _ref(W, st_type)
    wp = ostore.dequantize(ref["codes"], ref["absmax_q"], ref["absmax_s2"], N * K,
                           st_type).reshape(N, K)
    want = oracle.merge(wp, host_f32(A), host_f32(B), s)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want)  # oracle.merge returns the bf16 bit patterns
