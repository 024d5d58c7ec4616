"""qlora_linear_fwd_noalloc, the forward whose scratch memory is the
library's fixed per-device array, against qlora_linear_fwd with a caller
workspace: both run the same kernels, so Y and T must agree bit for bit.
Calls follow each other on one stream with shrinking inputs, so the second
call finds the array holding the first call's larger contents; both the
GEMV path (M <= 16) and the MFMA path are covered, and a path change
between calls."""

import pytest
import torch

import synthetic
from tests.gpu_util import device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    device()
    import bit_quantized_finetuning_quantize_amd as q
    return q


def _case(q, M, N, K, r, seed):
    dev = device()
    W, X, A, B, _ = synthetic.linear_inputs(M, N, K, r, dev, seed=seed, need_dy=False)
    st = q.qlora_nf4_quantize(W)
    return X, st, A, B, 2.0 / r


@pytest.mark.parametrize("shapes", [
    [(16, 4096, 4096, 16), (1, 256, 512, 8)],            # GEMV path, then a smaller GEMV
    [(2048, 11008, 4096, 64), (300, 384, 320, 16)],      # MFMA path, then a smaller MFMA
    [(4096, 8192, 8192, 64), (5, 192, 640, 3)],          # MFMA path, then the GEMV path
])
def test_noalloc_matches_workspace_call(q, shapes):
    cases = [_case(q, *sh, seed=sum(sh)) for sh in shapes]
    torch.cuda.synchronize()
    for (M, N, K, r), (X, st, A, B, s) in zip(shapes, cases):
        print(f"[case] noalloc M={M} N={N} K={K} r={r}", flush=True)
        Yn, Tn = q.qlora_linear_fwd_noalloc(X, st, A, B, s)
        Yw, Tw = q.qlora_linear_fwd(X, st, A, B, s)
        torch.cuda.synchronize()
        assert torch.equal(Yn, Yw), f"M={M} N={N} K={K} r={r}: Y differs from the workspace call"
        assert torch.equal(Tn, Tw), f"M={M} N={N} K={K} r={r}: T differs from the workspace call"
    # the same calls again in reverse order: the array now starts from the
    # smaller call's contents
    for (M, N, K, r), (X, st, A, B, s) in reversed(list(zip(shapes, cases))):
        Yn, Tn = q.qlora_linear_fwd_noalloc(X, st, A, B, s, want_T=False)
        Yw, _ = q.qlora_linear_fwd(X, st, A, B, s, want_T=False)
        torch.cuda.synchronize()
        assert torch.equal(Yn, Yw), f"repeat M={M} N={N} K={K} r={r}: Y differs"
