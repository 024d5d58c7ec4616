"""The decode forward (M <= 16) captured in a HIP graph: every replay, with
eager work and synchronizations between replays, must reproduce the eager
result bit for bit (the graph holds the same kernels on the same inputs)."""

import pytest
import torch

import synthetic
from tests.gpu_util import device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M", [1, 16])
def test_gemv_graph_replays_match_eager(M):
    dev = device()
    import bit_quantized_finetuning_quantize_amd as q
    N = K = 4096
    r, alpha = 16, 32
    print(f"[case] graph replay M={M} N={N} K={K} r={r}", flush=True)
    stores = []
    for i in range(3):
        W = synthetic.normal((N, K), 0.02, dev, 200 + i, synthetic.W_IDX)
        stores.append(q.qlora_nf4_quantize(W))
    A = synthetic.normal((K, r), 0.01, dev, 1, synthetic.A_IDX)
    B = synthetic.normal((r, N), 0.01, dev, 1, synthetic.B_IDX)
    X = synthetic.normal((M, K), 1.0, dev, 1, synthetic.X_IDX)
    ws = q.workspace(M, N, K, r, dev)
    eager = []
    for st in stores:
        Y, _ = q.qlora_linear_fwd(X, st, A, B, alpha / r, want_T=False, ws=ws)
        eager.append(Y.clone())
    Ys = [torch.empty(M, N, dtype=torch.bfloat16, device=dev) for _ in stores]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for st, Y in zip(stores, Ys):
            q.qlora_linear_fwd(X, st, A, B, alpha / r, want_T=False, Y=Y, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for st, Y in zip(stores, Ys):
            q.qlora_linear_fwd(X, st, A, B, alpha / r, want_T=False, Y=Y, ws=ws)
    for rep in range(4):
        for Y in Ys:
            Y.fill_(0)
        q.qlora_linear_fwd(X, stores[0], A, B, alpha / r, want_T=False, ws=ws)  # eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (Y, E) in enumerate(zip(Ys, eager)):
            assert torch.equal(Y, E), f"replay {rep}, call {i}: graph output differs from eager"
