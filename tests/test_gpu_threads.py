"""Calls from several host threads at once, each on its own stream with its
own workspace and buffers (the library keeps no per-call state; its only
process state, the raised LDS limit of a kernel, is set once per device
under an atomic flag): every thread's results equal those of the same calls
made one after another on one stream, bit for bit."""

import threading

import pytest
import torch

import synthetic
from tests.gpu_util import device

pytestmark = pytest.mark.gpu


def _work(q, dev, seed, M, N, K, r):
    W, X, A, B, dY = synthetic.linear_inputs(M, N, K, r, dev, seed=seed)
    return dict(W=W, X=X, A=A, B=B, dY=dY, M=M, N=N, K=K, r=r,
                ws=q.workspace(M, N, K, r, dev))


def _run(q, w, reps):
    outs = []
    for _ in range(reps):
        st = q.qlora_nf4_quantize(w["W"])
        Y, T = q.qlora_linear_fwd(w["X"], st, w["A"], w["B"], 0.5, ws=w["ws"])
        dX, dA, dB = q.qlora_linear_bwd(w["dY"], w["X"], T, st, w["A"], w["B"], 0.5, ws=w["ws"])
        outs.append((st.codes, Y, T, dX, dA, dB))
    return outs


def test_threads_on_separate_streams():
    dev = device()
    import bit_quantized_finetuning_quantize_amd as q
    shapes = [(300, 384, 320, 64), (8, 512, 256, 16), (512, 256, 512, 32), (4, 256, 256, 8)]
    print(f"[case] {len(shapes)} threads, shapes {shapes}", flush=True)
    works = [_work(q, dev, 40 + i, *sh) for i, sh in enumerate(shapes)]
    want = [_run(q, w, 1)[0] for w in works]
    torch.cuda.synchronize()
    results = [None] * len(works)
    errors = []

    def body(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                results[i] = _run(q, works[i], 6)
            s.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(e)

    threads = [threading.Thread(target=body, args=(i,)) for i in range(len(works))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i, outs in enumerate(results):
        for rep, got in enumerate(outs):
            for a, b in zip(got, want[i]):
                assert torch.equal(a, b), f"thread {i} repetition {rep} differs"
