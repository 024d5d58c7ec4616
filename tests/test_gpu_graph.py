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


@pytest.mark.parametrize("shape", [(300, 384, 320, 64), (64, 256, 512, 16)])
def test_training_step_graph_replays_match_eager(shape):
    """Every entry point in one captured step: quantize, dequantize, a dropout
    mask, forward and backward with and without dropout, the merge, and
    AdamW with float32 and with 8-bit state stepping copies of the adapter
    with dA and dB. The optimizer state is restored (eagerly) before each
    replay; every replay must equal the eager run bit for bit."""
    dev = device()
    import bit_quantized_finetuning_quantize_amd as q
    M, N, K, r = shape
    s, p = 2.0 / r * 16, 0.1
    print(f"[case] graph training step M={M} N={N} K={K} r={r}", flush=True)
    W, X, A, B, dY = synthetic.linear_inputs(M, N, K, r, dev, seed=31)
    st = q.empty_store(N * K, dev, (N, K))
    st1 = q.empty_store(N * K, dev, (N, K), double_quant=False)
    ws = q.workspace(M, N, K, r, dev)
    mask = torch.empty(M, K // 32, dtype=torch.int32, device=dev)
    bufs = dict(
        w32=torch.empty(N * K, dtype=torch.float32, device=dev),
        Y=torch.empty(M, N, dtype=torch.bfloat16, device=dev),
        T=torch.empty(M, r, dtype=torch.float32, device=dev),
        dX=torch.empty(M, K, dtype=torch.bfloat16, device=dev),
        dA=torch.empty(K, r, dtype=torch.float32, device=dev),
        dB=torch.empty(r, N, dtype=torch.float32, device=dev),
        Yd=torch.empty(M, N, dtype=torch.bfloat16, device=dev),
        Td=torch.empty(M, r, dtype=torch.float32, device=dev),
        dXd=torch.empty(M, K, dtype=torch.bfloat16, device=dev),
        dAd=torch.empty(K, r, dtype=torch.float32, device=dev),
        dBd=torch.empty(r, N, dtype=torch.float32, device=dev),
        merged=torch.empty(N, K, dtype=torch.bfloat16, device=dev),
        pa16=torch.empty(K * r, dtype=torch.bfloat16, device=dev),
        pb16=torch.empty(r * N, dtype=torch.bfloat16, device=dev),
    )
    # optimizer state: float32 for A's copy, 8-bit for B's copy
    pa0 = A.float().reshape(-1).clone()
    pb0 = B.float().reshape(-1).clone()
    state0 = dict(pa=pa0, ma=torch.zeros_like(pa0), va=torch.zeros_like(pa0), pb=pb0)
    m8, sm, v8, sv = q.adamw8_state(pb0.numel(), dev)
    state0.update(m8=m8, sm=sm, v8=v8, sv=sv)
    state = {k: v.clone() for k, v in state0.items()}

    def step():
        q.qlora_nf4_quantize(W, out=st)
        q.qlora_nf4_quantize(W, out=st1)
        q.qlora_nf4_dequantize(st1, out=bufs["w32"])
        q.qlora_dropout_mask(M, K, p, 77, 3, out=mask)
        q.qlora_linear_fwd(X, st, A, B, s, Y=bufs["Y"], T=bufs["T"], ws=ws)
        q.qlora_linear_bwd(dY, X, bufs["T"], st, A, B, s, dX=bufs["dX"], dA=bufs["dA"],
                           dB=bufs["dB"], ws=ws)
        q.qlora_linear_fwd_dropout(X, st1, A, B, s, mask, p, Y=bufs["Yd"], T=bufs["Td"], ws=ws)
        q.qlora_linear_bwd_dropout(dY, X, bufs["Td"], st1, A, B, s, mask, p, dX=bufs["dXd"],
                                   dA=bufs["dAd"], dB=bufs["dBd"], ws=ws)
        q.qlora_nf4_merge(st, A, B, s, out=bufs["merged"])
        q.qlora_adamw_step(state["pa"], state["ma"], state["va"], bufs["dAd"].reshape(-1), 2e-4,
                           step=1, weight_decay=0.01, p_bf16=bufs["pa16"])
        q.qlora_adamw8_step(state["pb"], state["m8"], state["sm"], state["v8"], state["sv"],
                            bufs["dBd"].reshape(-1), 2e-4, step=1, weight_decay=0.01,
                            p_bf16=bufs["pb16"])

    def snapshot():
        out = {k: v.clone() for k, v in bufs.items()}
        out.update({f"st_{i}": t.clone() for i, t in enumerate((st.codes, st.absmax_q, st.absmax_s2,
                                                               st1.codes, st1.absmax_s2, mask))})
        out.update({f"state_{k}": v.clone() for k, v in state.items()})
        return out

    def restore():
        for k, v in state0.items():
            state[k].copy_(v)

    step()
    torch.cuda.synchronize()
    eager = snapshot()
    restore()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        restore()
        for v in bufs.values():
            v.zero_()
        q.qlora_linear_fwd(X, st, A, B, s, ws=ws)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for k, v in eager.items():
            assert torch.equal(got[k], v), f"replay {rep}: {k} differs from eager"
