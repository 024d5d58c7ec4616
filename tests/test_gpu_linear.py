"""GPU forward / backward parity against the oracle (bf16 compute, float32
accumulation): max |gpu - oracle| / max |oracle| <= 2e-2 for Y, dX, dA, dB,
plus exact special cases, determinism and the full-size prefill projection."""

import numpy as np
import pytest
import torch

import oracle
import synthetic
from tests.gpu_util import TOL, assert_close, assert_store_equal, device, host_f32, oracle_wprime

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    device()
    import bit_quantized_finetuning_quantize_amd as q
    return q


def _run(q, M, N, K, r, alpha, seed=0, weight="normal", bwd=True, zero=None, label=None):
    dev = device()
    label = label or f"M={M} N={N} K={K} r={r}"
    print(f"[case] {label}", flush=True)
    W, X, A, B, dY = synthetic.linear_inputs(M, N, K, r, dev, seed=seed, weight=weight,
                                             need_dy=bwd)
    if zero == "W":
        W = torch.zeros_like(W)
    elif zero == "A":
        A = torch.zeros_like(A)
    elif zero == "B":
        B = torch.zeros_like(B)
    s = alpha / r
    st = q.qlora_nf4_quantize(W)
    Y, T = q.qlora_linear_fwd(X, st, A, B, s)
    out = {"Y": Y, "T": T}
    if bwd:
        dX, dA, dB = q.qlora_linear_bwd(dY, X, T, st, A, B, s)
        out.update(dX=dX, dA=dA, dB=dB)
    torch.cuda.synchronize()
    ref, wp = oracle_wprime(W)
    assert_store_equal(st, ref, label)
    Xh, Ah, Bh = host_f32(X), host_f32(A), host_f32(B)
    Yo, To = oracle.linear_fwd(Xh, wp, Ah, Bh, s)
    res = {"Y": assert_close(host_f32(Y), Yo, label + " Y"),
           "T": assert_close(host_f32(T), To, label + " T", tol=1e-5)}
    if bwd:
        dXo, dAo, dBo = oracle.linear_bwd(host_f32(dY), Xh, wp, Ah, Bh, s)
        res["dX"] = assert_close(host_f32(out["dX"]), dXo, label + " dX")
        res["dA"] = assert_close(host_f32(out["dA"]), dAo, label + " dA") if np.any(dAo) else None
        res["dB"] = assert_close(host_f32(out["dB"]), dBo, label + " dB") if np.any(dBo) else None
    return out, res


def test_single_256(q):
    """The 256x256 workload: M=16, r=8, alpha=16 (GEMV forward path)."""
    _run(q, 16, 256, 256, 8, 16, label="single 256x256 M=16 r=8")


@pytest.mark.parametrize("M", [1, 4, 16])
def test_decode_gemv_4096(q, M):
    _run(q, M, 4096, 4096, 16, 32, bwd=False, label=f"decode 4096^2 M={M} r=16")


@pytest.mark.parametrize("M", [1, 16])
def test_decode_gemv_down_projection(q, M):
    """The GEMV on the 4096x11008 down projection: K = 11008 spans three
    4096-wide passes (the last one partial, ending inside a wave's range),
    and K / 64 = 172 blocks per row, so rows do not start on an eight-block
    boundary and a lane's blocks may straddle a second-level group."""
    _run(q, M, 4096, 11008, 16, 32, bwd=False, label=f"decode 4096x11008 M={M} r=16")


@pytest.mark.parametrize("shape", [
    (1, 256, 640, 6),         # short adapter rows (6 ranks)
    (1, 256, 640, 3),         # an odd rank: adapter rows off a 4-byte boundary
    (2, 192, 4160, 16),       # a second, partial 4096-wide pass
    (3, 320, 64, 8),          # one block of K
    (4, 128, 8256, 13),       # three passes, the last one partial, odd rank
])
@pytest.mark.parametrize("zero", [None, "W"])
def test_decode_small_ranks(q, shape, zero):
    """The small-M path at M <= 4 with ranks below 16 and K over partial
    4096-wide passes; with W = 0, Y is the adapter term alone."""
    M, N, K, r = shape
    _run(q, M, N, K, r, 2 * r, seed=M * 7 + r, bwd=False, zero=zero,
         label=f"small-M M={M} N={N} K={K} r={r}" + (" W=0" if zero else ""))


@pytest.mark.parametrize("shape", [
    (17, 256, 256, 8),        # just above the GEMV limit
    (300, 320, 192, 16),      # ragged M, N not a multiple of 128, K % 128 = 64
    (256, 128, 128, 64),      # exactly one tile
    (513, 384, 448, 100),     # r not a multiple of 64 (padded to 128)
    (64, 64, 64, 1),          # rank 1
    (5, 192, 640, 3),         # tiny M on the GEMV path with odd rank
])
def test_ragged_shapes(q, shape):
    M, N, K, r = shape
    _run(q, M, N, K, r, 2 * r, seed=M + N + K)


@pytest.mark.parametrize("shape", [
    (300, 256, 320, 256),     # the largest rank: four LoRA steps on the MFMA paths
    (200, 192, 256, 129),     # an odd rank padded to 192
    (4, 256, 512, 256),       # the largest rank on the GEMV path
    (16, 384, 256, 200),
])
@pytest.mark.parametrize("zero", [None, "W"])
def test_large_ranks(q, shape, zero):
    """Ranks up to the limit, with the workload's adapters and with W = 0
    (where Y and dX are the adapter terms alone)."""
    M, N, K, r = shape
    _run(q, M, N, K, r, 2 * r, seed=M + r, zero=zero,
         label=f"M={M} N={N} K={K} r={r}" + (" W=0" if zero else ""))


@pytest.mark.parametrize("M", [8, 96])
def test_adapter_only_when_weight_is_zero(q, M):
    """W = 0: Y is exactly the adapter term, so the LoRA path is checked at
    full relative strength (it is ~1% of Y otherwise)."""
    out, res = _run(q, M, 256, 512, 16, 64, zero="W", label=f"W=0 M={M}")


def test_zero_adapter_gradients(q):
    out, _ = _run(q, 96, 256, 256, 8, 16, zero="B", label="B=0")
    assert torch.count_nonzero(out["dA"]).item() == 0
    out, _ = _run(q, 96, 256, 256, 8, 16, zero="A", label="A=0")
    assert torch.count_nonzero(out["dB"]).item() == 0


def test_deterministic_and_T_recompute(q):
    dev = device()
    M, N, K, r = 300, 384, 256, 16
    W, X, A, B, dY = synthetic.linear_inputs(M, N, K, r, dev, seed=11)
    st = q.qlora_nf4_quantize(W)
    Y1, T1 = q.qlora_linear_fwd(X, st, A, B, 1.0)
    Y2, T2 = q.qlora_linear_fwd(X, st, A, B, 1.0)
    g1 = q.qlora_linear_bwd(dY, X, T1, st, A, B, 1.0)
    g2 = q.qlora_linear_bwd(dY, X, None, st, A, B, 1.0)  # T recomputed
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2) and torch.equal(T1, T2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_outputs_at_two_byte_offsets(q):
    """Y and dX written at a 2-byte offset (allowed: the outputs need only
    2-byte alignment): the contraction kernels then store their bf16 tiles
    element by element instead of in 16-byte row chunks. The values must be
    those of the aligned call, bit for bit, with nothing written outside
    the outputs."""
    dev = device()
    M, N, K, r = 300, 320, 192, 16
    print(f"[case] unaligned outputs M={M} N={N} K={K} r={r}", flush=True)
    W, X, A, B, dY = synthetic.linear_inputs(M, N, K, r, dev, seed=21)
    st = q.qlora_nf4_quantize(W)
    Y1, T1 = q.qlora_linear_fwd(X, st, A, B, 0.5)
    dX1, dA1, dB1 = q.qlora_linear_bwd(dY, X, T1, st, A, B, 0.5)
    sentinel = -7
    ybuf = torch.full((M * N + 2,), sentinel, dtype=torch.int16, device=dev)
    xbuf = torch.full((M * K + 2,), sentinel, dtype=torch.int16, device=dev)
    Y2 = ybuf[1:1 + M * N].view(torch.bfloat16).view(M, N)
    dX2 = xbuf[1:1 + M * K].view(torch.bfloat16).view(M, K)
    assert Y2.data_ptr() % 16 != 0 and dX2.data_ptr() % 16 != 0
    _, T2 = q.qlora_linear_fwd(X, st, A, B, 0.5, Y=Y2)
    _, dA2, dB2 = q.qlora_linear_bwd(dY, X, T2, st, A, B, 0.5, dX=dX2)
    torch.cuda.synchronize()
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))
    assert torch.equal(dX1.view(torch.int16), dX2.view(torch.int16))
    assert torch.equal(T1, T2) and torch.equal(dA1, dA2) and torch.equal(dB1, dB2)
    for buf, n in ((ybuf, M * N), (xbuf, M * K)):
        assert buf[0].item() == sentinel and buf[n + 1].item() == sentinel


def test_prefill_projection_full(q):
    """One full-size projection of the prefill MLP workload:
    gate W 11008x4096, X 2048x4096, r=64, alpha=16, compared in full."""
    _run(q, 2048, 11008, 4096, 64, 16, label="prefill gate 11008x4096 M=2048")


def test_prefill_down_projection_sampled(q):
    """down W 4096x11008 (contraction 11008): Y and dX on sampled rows,
    dA and dB in full."""
    dev = device()
    M, N, K, r, s = 2048, 4096, 11008, 64, 16 / 64
    W, X, A, B, dY = synthetic.linear_inputs(M, N, K, r, dev, seed=0, base=16)
    st = q.qlora_nf4_quantize(W)
    Y, T = q.qlora_linear_fwd(X, st, A, B, s)
    dX, dA, dB = q.qlora_linear_bwd(dY, X, T, st, A, B, s)
    torch.cuda.synchronize()
    ref, wp = oracle_wprime(W)
    assert_store_equal(st, ref, "down")
    rows = np.sort(np.random.default_rng(0).choice(M, 64, replace=False))
    Xh, Ah, Bh, dYh = host_f32(X), host_f32(A), host_f32(B), host_f32(dY)
    Yo, _ = oracle.linear_fwd(Xh[rows], wp, Ah, Bh, s)
    assert_close(host_f32(Y)[rows], Yo, "down Y rows")
    dXo, _, _ = oracle.linear_bwd(dYh[rows], Xh[rows], wp, Ah, Bh, s)
    assert_close(host_f32(dX)[rows], dXo, "down dX rows")
    _, dAo, dBo = oracle.linear_bwd(dYh, Xh, np.zeros((N, K), np.float32), Ah, Bh, s)
    assert_close(host_f32(dA), dAo, "down dA")
    assert_close(host_f32(dB), dBo, "down dB")


@pytest.mark.parametrize("M,N,K", [(16, 256, 512), (64, 384, 320), (160, 192, 640)])
def test_compute_weight_bit_exact_in_products(q, M, N, K):
    """One-hot token rows and a zero adapter make every output a single
    product 1 * bf16(w'): the forward returns Y[m][n] = bf16(w'[n][k_m]) and
    dX with one-hot dY rows returns bf16(w'[n_m][k]) exactly. This pins the
    dequantization inside the fused kernels (GEMV for M <= 16, the MFMA
    contraction otherwise) bit for bit to the oracle's compute weight."""
    dev = device()
    print(f"[case] one-hot compute weight M={M} N={N} K={K}", flush=True)
    r = 8
    W, _, _, _, _ = synthetic.linear_inputs(M, N, K, r, dev, seed=3, need_dy=False)
    st = q.qlora_nf4_quantize(W)
    ref, wp = oracle_wprime(W)
    wpb = oracle.bf16_round(wp)  # bf16(w') as float values
    rng = np.random.default_rng(M + N + K)
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
    Yh, dXh = host_f32(Y), host_f32(dX)
    np.testing.assert_array_equal(Yh, wpb[:, ks].T.astype(np.float32), err_msg="forward weights")
    np.testing.assert_array_equal(dXh, wpb[ns, :].astype(np.float32), err_msg="dX weights")
