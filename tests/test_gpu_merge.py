"""GPU adapter merge (qlora_nf4_merge) against the oracle: bit-exact bf16
merged weights, ragged row counts, ranks that are not multiples of the
kernel's rank chunk, the zero-adapter case and a sampled full-size case."""

import numpy as np
import pytest
import torch

import oracle
import synthetic
from oracle.bf16 import f32_to_bf16_bits
from tests.gpu_util import device, host_f32, store_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    device()
    import bit_quantized_finetuning_quantize_amd as q
    return q


def _bits(t):
    torch.cuda.synchronize()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _inputs(N, K, r, seed):
    dev = device()
    W = synthetic.normal((N, K), 0.02, dev, seed, synthetic.W_IDX)
    A = synthetic.normal((K, r), 0.01, dev, seed, synthetic.A_IDX)
    B = synthetic.normal((r, N), 0.01, dev, seed, synthetic.B_IDX)
    return W, A, B


def _oracle_merge(st, N, K, A, B, scale, rows=None):
    codes, q8, s2 = store_np(st)
    wp = oracle.dequantize(codes, q8, s2, N * K).reshape(N, K)
    Ah, Bh = host_f32(A), host_f32(B)
    if rows is not None:
        wp, Bh = wp[rows], Bh[:, rows]
    return oracle.merge(wp, Ah, Bh, scale)


@pytest.mark.parametrize("N,K,r,scale", [
    (64, 64, 8, 2.0),        # one tile
    (100, 128, 16, 0.25),    # ragged rows
    (256, 512, 64, 0.25),    # several tiles, two rank chunks
    (192, 256, 40, 0.37),    # rank not a multiple of the 32-rank chunk
    (65, 192, 1, 1.0),       # rank one, one row past a tile
    (128, 128, 256, 0.0625), # the largest rank: eight rank chunks
    (96, 320, 129, 0.5),     # a chunk of one rank at the end
])
def test_merge_bit_exact(q, N, K, r, scale):
    print(f"[case] merge N={N} K={K} r={r} s={scale}", flush=True)
    W, A, B = _inputs(N, K, r, seed=N + K + r)
    st = q.qlora_nf4_quantize(W)
    got = _bits(q.qlora_nf4_merge(st, A, B, scale))
    want = _oracle_merge(st, N, K, A, B, scale)
    assert np.array_equal(got, want), f"{np.sum(got != want)} of {got.size} differ"


def test_zero_adapter_equals_bf16_dequantize(q):
    N, K, r = 128, 256, 16
    W, A, B = _inputs(N, K, r, seed=3)
    st = q.qlora_nf4_quantize(W)
    got = _bits(q.qlora_nf4_merge(st, torch.zeros_like(A), B, 0.25))
    want = _bits(q.qlora_nf4_dequantize_bf16(st)).reshape(N, K)
    assert np.array_equal(got, want)


def test_merge_full_size_sampled(q):
    """11008 x 4096, r = 64 (the gate projection's shape), 96 sampled rows
    spread over the row tiles; every output finite; two calls identical."""
    N, K, r, scale = 11008, 4096, 64, 0.25
    print(f"[case] merge N={N} K={K} r={r} sampled", flush=True)
    W, A, B = _inputs(N, K, r, seed=11)
    st = q.qlora_nf4_quantize(W)
    out = q.qlora_nf4_merge(st, A, B, scale)
    again = q.qlora_nf4_merge(st, A, B, scale)
    got = _bits(out)
    assert np.array_equal(got, _bits(again))
    assert torch.isfinite(out.float()).all().item()
    rng = np.random.default_rng(0)
    rows = np.sort(np.concatenate([rng.choice(N, 90, replace=False), [0, 63, 64, N - 65, N - 2, N - 1]]))
    want = _oracle_merge(st, N, K, A, B, scale, rows=rows)
    assert np.array_equal(got[rows], want)
