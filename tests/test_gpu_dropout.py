"""GPU parity of LoRA dropout against the oracle.

  * the keep mask bit for bit (shapes, probabilities, 64-bit seeds and
    offsets, the full-size prefill inputs);
  * forward and backward with the mask: T at 1e-5, Y, dX, dA, dB at the
    linear layer's tolerance (max |gpu - oracle| / max |oracle| <= 2e-2);
    with a zero frozen weight so that Y and dX consist of the masked adapter
    terms alone (with the workload's adapter scale they are far below the
    tolerance next to the frozen-weight product);
  * p = 0 reproduces the plain path (bit for bit where the kernels are the
    same, within the tolerance for dX, whose adapter columns are summed
    apart), T recomputed in the backward gives the same gradients bit for
    bit, the rank limit of the masked input gradient;
  * the full-size prefill projections (gate 11008x4096 in full, down
    4096x11008 on sampled rows) and the 65B-shaped down projection
    (8192x22016, 4096 tokens) on sampled rows.
"""

import numpy as np
import pytest
import torch

import oracle
import synthetic
from tests.gpu_util import TOL, assert_close, device, host_f32, oracle_wprime

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    device()
    import bit_quantized_finetuning_quantize_amd as q
    return q


def _mask_np(mask):
    return mask.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("M,K,p,seed,offset", [
    (1, 64, 0.05, 0, 0),
    (7, 192, 0.05, 1, 0),
    (300, 320, 0.1, 12345, 3),
    (64, 4096, 0.5, (1 << 40) + 17, (1 << 33) + 5),
    (33, 256, 0.0, 9, 0),
    (128, 128, 0.999, 2, 1),
])
def test_mask_bit_exact(q, M, K, p, seed, offset):
    print(f"[case] mask M={M} K={K} p={p} seed={seed} offset={offset}", flush=True)
    got = _mask_np(q.qlora_dropout_mask(M, K, p, seed, offset, device=device()))
    torch.cuda.synchronize()
    want = oracle.pack_keep(oracle.dropout_keep(M, K, p, seed, offset))
    assert np.array_equal(got, want)


def test_mask_full_size(q):
    """The down projection's input, 2048 x 11008, p = 0.05."""
    M, K = 2048, 11008
    print(f"[case] mask M={M} K={K} full", flush=True)
    got = _mask_np(q.qlora_dropout_mask(M, K, 0.05, 2024, 7, device=device()))
    torch.cuda.synchronize()
    want = oracle.pack_keep(oracle.dropout_keep(M, K, 0.05, 2024, 7))
    assert np.array_equal(got, want)


def _run(q, M, N, K, r, alpha, p, seed=0, zero_w=False, label=None, T_given=True, dq=True):
    dev = device()
    label = label or f"M={M} N={N} K={K} r={r} p={p}" + (" W=0" if zero_w else "") + \
        ("" if dq else " no DQ")
    print(f"[case] dropout {label}", flush=True)
    W, X, A, B, dY = synthetic.linear_inputs(M, N, K, r, dev, seed=seed)
    if zero_w:
        W = torch.zeros_like(W)
    s = alpha / r
    mask = q.qlora_dropout_mask(M, K, p, seed + 101, 5, device=dev)
    st = q.qlora_nf4_quantize(W, double_quant=dq)
    Y, T = q.qlora_linear_fwd_dropout(X, st, A, B, s, mask, p)
    dX, dA, dB = q.qlora_linear_bwd_dropout(dY, X, T if T_given else None, st, A, B, s, mask, p)
    torch.cuda.synchronize()
    keep = oracle.dropout_keep(M, K, p, seed + 101, 5)
    assert np.array_equal(_mask_np(mask), oracle.pack_keep(keep)), label + " mask"
    ks = oracle.keep_scale(p)
    if dq:
        _, wp = oracle_wprime(W)
    else:
        ref = oracle.quantize(host_f32(W).ravel())
        wp = oracle.dequantize_nodq(ref["codes"], ref["absmax"], N * K).reshape(N, K)
    Xh, Ah, Bh, dYh = host_f32(X), host_f32(A), host_f32(B), host_f32(dY)
    Yo, To = oracle.linear_fwd(Xh, wp, Ah, Bh, s, keep=keep, keep_scale=ks)
    dXo, dAo, dBo = oracle.linear_bwd(dYh, Xh, wp, Ah, Bh, s, keep=keep, keep_scale=ks)
    assert_close(host_f32(T), To, label + " T", tol=1e-5)
    assert_close(host_f32(Y), Yo, label + " Y")
    assert_close(host_f32(dX), dXo, label + " dX")
    assert_close(host_f32(dA), dAo, label + " dA")
    assert_close(host_f32(dB), dBo, label + " dB")
    return dict(Y=Y, T=T, dX=dX, dA=dA, dB=dB, mask=mask, st=st, X=X, A=A, B=B, dY=dY, s=s)


SHAPES = [
    (256, 128, 128, 64),      # one tile
    (300, 320, 192, 16),      # ragged M, K % 128 = 64: the last column tile half past K
    (513, 384, 448, 100),     # r padded to 128: two LoRA steps, padded adapter copies
    (1, 256, 256, 8),         # one token (the MFMA path serves every M under dropout)
    (16, 256, 256, 8),
    (200, 192, 640, 192),     # the largest rank of the masked input gradient: three steps
]


@pytest.mark.parametrize("shape", SHAPES)
def test_dropout_parity(q, shape):
    M, N, K, r = shape
    _run(q, M, N, K, r, 2 * r, 0.05, seed=M + N + K)


@pytest.mark.parametrize("shape", SHAPES)
def test_dropout_parity_zero_weight(q, shape):
    """W = 0: Y = s D(X) A B and dX = s ((G A^T) o keep) f, nothing else."""
    M, N, K, r = shape
    _run(q, M, N, K, r, 2 * r, 0.3, seed=M + 2 * N + K, zero_w=True)


@pytest.mark.parametrize("shape", [(300, 320, 192, 16), (16, 256, 256, 8)])
def test_dropout_on_store_without_double_quant(q, shape):
    M, N, K, r = shape
    _run(q, M, N, K, r, 2 * r, 0.1, seed=M + N, dq=False)


def test_p_zero_matches_plain_path(q):
    dev = device()
    M, N, K, r, s = 300, 384, 320, 64, 0.25
    print(f"[case] dropout p=0 vs plain M={M} N={N} K={K} r={r}", flush=True)
    W, X, A, B, dY = synthetic.linear_inputs(M, N, K, r, dev, seed=21)
    st = q.qlora_nf4_quantize(W)
    mask = q.qlora_dropout_mask(M, K, 0.0, 1, 0, device=dev)
    Y0, T0 = q.qlora_linear_fwd(X, st, A, B, s)
    Y1, T1 = q.qlora_linear_fwd_dropout(X, st, A, B, s, mask, 0.0)
    g0 = q.qlora_linear_bwd(dY, X, T0, st, A, B, s)
    g1 = q.qlora_linear_bwd_dropout(dY, X, T1, st, A, B, s, mask, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(Y0, Y1) and torch.equal(T0, T1)
    assert torch.equal(g0[1], g1[1]) and torch.equal(g0[2], g1[2])
    assert_close(host_f32(g1[0]), host_f32(g0[0]), "p=0 dX vs plain", tol=1e-2)


def test_T_recompute_and_determinism(q):
    dev = device()
    M, N, K, r, s, p = 300, 256, 384, 16, 1.0, 0.2
    print(f"[case] dropout T recompute M={M} N={N} K={K} r={r}", flush=True)
    W, X, A, B, dY = synthetic.linear_inputs(M, N, K, r, dev, seed=5)
    st = q.qlora_nf4_quantize(W)
    mask = q.qlora_dropout_mask(M, K, p, 77, 0, device=dev)
    Y1, T1 = q.qlora_linear_fwd_dropout(X, st, A, B, s, mask, p)
    Y2, T2 = q.qlora_linear_fwd_dropout(X, st, A, B, s, mask, p)
    g1 = q.qlora_linear_bwd_dropout(dY, X, T1, st, A, B, s, mask, p)
    g2 = q.qlora_linear_bwd_dropout(dY, X, None, st, A, B, s, mask, p)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2) and torch.equal(T1, T2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_rank_limit_of_masked_input_gradient(q):
    dev = device()
    M, N, K, r, s, p = 64, 128, 128, 256, 0.1, 0.05
    print(f"[case] dropout r={r} limit", flush=True)
    W, X, A, B, dY = synthetic.linear_inputs(M, N, K, r, dev, seed=8)
    st = q.qlora_nf4_quantize(W)
    mask = q.qlora_dropout_mask(M, K, p, 3, 0, device=dev)
    Y, T = q.qlora_linear_fwd_dropout(X, st, A, B, s, mask, p)
    with pytest.raises(q.QloraError):
        q.qlora_linear_bwd_dropout(dY, X, T, st, A, B, s, mask, p)
    # without the input gradient every rank is served
    _, dA, dB = q.qlora_linear_bwd_dropout(dY, X, T, st, A, B, s, mask, p, want_dX=False)
    torch.cuda.synchronize()
    keep = oracle.dropout_keep(M, K, p, 3, 0)
    ks = oracle.keep_scale(p)
    _, wp = oracle_wprime(W)
    Xh, Ah, Bh, dYh = host_f32(X), host_f32(A), host_f32(B), host_f32(dY)
    Yo, To = oracle.linear_fwd(Xh, wp, Ah, Bh, s, keep=keep, keep_scale=ks)
    _, dAo, dBo = oracle.linear_bwd(dYh, Xh, wp, Ah, Bh, s, keep=keep, keep_scale=ks)
    assert_close(host_f32(T), To, "r=256 T", tol=1e-5)
    assert_close(host_f32(Y), Yo, "r=256 Y")
    assert_close(host_f32(dA), dAo, "r=256 dA")
    assert_close(host_f32(dB), dBo, "r=256 dB")


def test_prefill_gate_full(q):
    """gate W 11008x4096, X 2048x4096, r=64, alpha=16, p=0.05, in full."""
    _run(q, 2048, 11008, 4096, 64, 16, 0.05, label="prefill gate 11008x4096 M=2048 p=0.05")


def test_prefill_down_sampled(q):
    """down W 4096x11008 (contraction 11008), p = 0.05: T, Y and dX on
    sampled rows, dA and dB in full."""
    dev = device()
    M, N, K, r, s, p = 2048, 4096, 11008, 64, 16 / 64, 0.05
    print("[case] dropout prefill down 4096x11008 M=2048", flush=True)
    W, X, A, B, dY = synthetic.linear_inputs(M, N, K, r, dev, seed=0, base=16)
    st = q.qlora_nf4_quantize(W)
    mask = q.qlora_dropout_mask(M, K, p, 99, 1, device=dev)
    Y, T = q.qlora_linear_fwd_dropout(X, st, A, B, s, mask, p)
    dX, dA, dB = q.qlora_linear_bwd_dropout(dY, X, T, st, A, B, s, mask, p)
    torch.cuda.synchronize()
    keep = oracle.dropout_keep(M, K, p, 99, 1)
    assert np.array_equal(_mask_np(mask), oracle.pack_keep(keep))
    ks = oracle.keep_scale(p)
    _, wp = oracle_wprime(W)
    rows = np.sort(np.random.default_rng(1).choice(M, 64, replace=False))
    Xh, Ah, Bh, dYh = host_f32(X), host_f32(A), host_f32(B), host_f32(dY)
    Yo, To = oracle.linear_fwd(Xh[rows], wp, Ah, Bh, s, keep=keep[rows], keep_scale=ks)
    assert_close(host_f32(T)[rows], To, "down T rows", tol=1e-5)
    assert_close(host_f32(Y)[rows], Yo, "down Y rows")
    dXo, _, _ = oracle.linear_bwd(dYh[rows], Xh[rows], wp, Ah, Bh, s, keep=keep[rows],
                                  keep_scale=ks)
    assert_close(host_f32(dX)[rows], dXo, "down dX rows")
    _, dAo, dBo = oracle.linear_bwd(dYh, Xh, np.zeros((N, K), np.float32), Ah, Bh, s, keep=keep,
                                    keep_scale=ks)
    assert_close(host_f32(dA), dAo, "down dA")
    assert_close(host_f32(dB), dBo, "down dB")


def test_stress_down_projection_sampled(q):
    """The 65B-shaped down projection (W 8192x22016, Student-t weights),
    4096 tokens, p = 0.05: the mask in full, T, Y and dX on sampled rows,
    dA and dB in full."""
    dev = device()
    M, N, K, r, s, p = 4096, 8192, 22016, 64, 16 / 64, 0.05
    print("[case] dropout stress down 8192x22016 M=4096", flush=True)
    W, X, A, B, dY = synthetic.linear_inputs(M, N, K, r, dev, seed=2, weight="student_t")
    st = q.qlora_nf4_quantize(W)
    mask = q.qlora_dropout_mask(M, K, p, 5150, 11, device=dev)
    Y, T = q.qlora_linear_fwd_dropout(X, st, A, B, s, mask, p)
    dX, dA, dB = q.qlora_linear_bwd_dropout(dY, X, T, st, A, B, s, mask, p)
    torch.cuda.synchronize()
    keep = oracle.dropout_keep(M, K, p, 5150, 11)
    assert np.array_equal(_mask_np(mask), oracle.pack_keep(keep))
    ks = oracle.keep_scale(p)
    rows = np.sort(np.random.default_rng(2).choice(M, 24, replace=False))
    _, wp = oracle_wprime(W)
    Xh, Ah, Bh, dYh = host_f32(X), host_f32(A), host_f32(B), host_f32(dY)
    Yo, To = oracle.linear_fwd(Xh[rows], wp, Ah, Bh, s, keep=keep[rows], keep_scale=ks)
    assert_close(host_f32(T)[rows], To, "stress down T rows", tol=1e-5)
    assert_close(host_f32(Y)[rows], Yo, "stress down Y rows")
    dXo, _, _ = oracle.linear_bwd(dYh[rows], Xh[rows], wp, Ah, Bh, s, keep=keep[rows],
                                  keep_scale=ks)
    assert_close(host_f32(dX)[rows], dXo, "stress down dX rows")
    _, dAo, dBo = oracle.linear_bwd(dYh, Xh, np.zeros((N, K), np.float32), Ah, Bh, s, keep=keep,
                                    keep_scale=ks)
    assert_close(host_f32(dA), dAo, "stress down dA")
    assert_close(host_f32(dB), dBo, "stress down dB")
