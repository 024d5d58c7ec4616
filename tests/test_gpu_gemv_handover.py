"""The small-M forward's one launch: workgroups that form T = X A hand it to
the row-tile workgroups through a flag tagged with the dispatch. These tests
check that the handover is exact: with the wait switched off (every row-tile
workgroup forms T itself) the outputs are the same bit for bit; a single
captured call replayed on new inputs, back-to-back calls on one workspace,
and calls alternating between two streams on one workspace all give what
each call gives alone."""

import pytest
import torch

import oracle
import synthetic
from tests.gpu_util import assert_close, device, host_f32, oracle_wprime

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    device()
    import bit_quantized_finetuning_quantize_amd as q
    yield q
    q.qlora_gemv_wait_limit(200)


@pytest.mark.parametrize("shape", [
    (1, 4096, 4096, 16),
    (4, 4096, 4096, 16),
    (16, 4096, 4096, 16),
    (16, 4096, 11008, 64),   # three passes, four adapter column groups
    (3, 320, 64, 8),         # one block of K
    (2, 192, 4160, 3),       # an odd rank, a partial second pass
    (16, 256, 4096, 256),    # the largest rank: T in the token rows' LDS
])
def test_wait_off_gives_the_same_bits(q, shape):
    M, N, K, r = shape
    dev = device()
    print(f"[case] handover vs in-workgroup T M={M} N={N} K={K} r={r}", flush=True)
    W, X, A, B, _ = synthetic.linear_inputs(M, N, K, r, dev, seed=7, need_dy=False)
    st = q.qlora_nf4_quantize(W)
    s = 2.0
    try:
        q.qlora_gemv_wait_limit(200)
        Y1, T1 = q.qlora_linear_fwd(X, st, A, B, s)
        q.qlora_gemv_wait_limit(0)
        Y0, T0 = q.qlora_linear_fwd(X, st, A, B, s)
        torch.cuda.synchronize()
    finally:
        q.qlora_gemv_wait_limit(200)
    assert torch.equal(Y0, Y1), "Y differs between the handover and the in-workgroup T"
    assert torch.equal(T0, T1), "T differs between the handover and the in-workgroup T"
    if N * K <= 4096 * 4160:
        _, wp = oracle_wprime(W)
        Yo, To = oracle.linear_fwd(host_f32(X), wp, host_f32(A), host_f32(B), s)
        assert_close(host_f32(Y0), Yo, "Y")
        assert_close(host_f32(T0), To, "T", tol=1e-5)


def _inputs(q, M, N, K, r, n, dev):
    out = []
    for i in range(n):
        W = synthetic.normal((N, K), 0.02, dev, 300 + i, synthetic.W_IDX)
        X = synthetic.normal((M, K), 1.0, dev, 400 + i, synthetic.X_IDX)
        A = synthetic.normal((K, r), 0.01, dev, 500 + i, synthetic.A_IDX)
        B = synthetic.normal((r, N), 0.01, dev, 600 + i, synthetic.B_IDX)
        out.append((q.qlora_nf4_quantize(W), X, A, B))
    return out


def _alone(q, data, ws, s):
    ref = []
    for st, X, A, B in data:
        Y, T = q.qlora_linear_fwd(X, st, A, B, s, ws=ws)
        torch.cuda.synchronize()
        ref.append((Y.clone(), T.clone()))
    return ref


@pytest.mark.parametrize("M", [1, 16])
def test_one_call_graph_on_new_inputs(q, M):
    """One captured call, replayed after its input tensors are overwritten:
    the replay must not take T's partials or flags of an earlier replay."""
    dev = device()
    N = K = 4096
    r, s = 16, 2.0
    print(f"[case] one-call graph, new inputs per replay, M={M}", flush=True)
    data = _inputs(q, M, N, K, r, 5, dev)
    ws = q.workspace(M, N, K, r, dev)
    st0, X0, A0, B0 = data[0]
    X, A = X0.clone(), A0.clone()
    Y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    T = torch.empty(M, r, dtype=torch.float32, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        q.qlora_linear_fwd(X, st0, A, B0, s, Y=Y, T=T, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        q.qlora_linear_fwd(X, st0, A, B0, s, Y=Y, T=T, ws=ws)
    for rep in range(3):
        for i, (_, Xi, Ai, _) in enumerate(data):
            # the same store and B, new tokens and adapter A
            X.copy_(Xi)
            A.copy_(Ai)
            Ye, Te = q.qlora_linear_fwd(X, st0, A, B0, s)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(Y, Ye), f"replay {rep} input {i}: Y differs from the eager call"
            assert torch.equal(T, Te), f"replay {rep} input {i}: T differs from the eager call"


@pytest.mark.parametrize("M", [1, 4, 16])
def test_back_to_back_calls_on_one_workspace(q, M):
    dev = device()
    N = K = 4096
    r, s = 16, 2.0
    print(f"[case] back-to-back calls on one workspace, M={M}", flush=True)
    data = _inputs(q, M, N, K, r, 24, dev)
    ws = q.workspace(M, N, K, r, dev)
    ref = _alone(q, data, ws, s)
    for rep in range(2):
        got = [q.qlora_linear_fwd(X, st, A, B, s, ws=ws) for st, X, A, B in data]
        torch.cuda.synchronize()
        for i, ((Y, T), (Yr, Tr)) in enumerate(zip(got, ref)):
            assert torch.equal(Y, Yr), f"rep {rep} call {i}: Y differs from the call alone"
            assert torch.equal(T, Tr), f"rep {rep} call {i}: T differs from the call alone"


def test_calls_alternating_between_two_streams(q):
    """Calls on one workspace issued alternately on two streams, each call
    ordered after the previous one by an event: the tag of a dispatch on one
    queue must never match a flag left by the other."""
    dev = device()
    M, N, K, r, s = 4, 4096, 4096, 16, 2.0
    print("[case] two streams, one workspace", flush=True)
    data = _inputs(q, M, N, K, r, 16, dev)
    ws = q.workspace(M, N, K, r, dev)
    ref = _alone(q, data, ws, s)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    got = []
    prev = torch.cuda.current_stream()
    for i, (st, X, A, B) in enumerate(data):
        cur = streams[i % 2]
        cur.wait_stream(prev)
        with torch.cuda.stream(cur):
            got.append(q.qlora_linear_fwd(X, st, A, B, s, ws=ws))
        prev = cur
    torch.cuda.current_stream().wait_stream(prev)
    torch.cuda.synchronize()
    for i, ((Y, T), (Yr, Tr)) in enumerate(zip(got, ref)):
        assert torch.equal(Y, Yr), f"call {i}: Y differs from the call alone"
        assert torch.equal(T, Tr), f"call {i}: T differs from the call alone"
