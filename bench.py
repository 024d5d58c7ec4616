#!/usr/bin/env python3
"""Benchmark of the NF4 linear layer with a LoRA adapter on one MI355X.

Primary line: fwd+bwd TFLOP/s on the prefill-shaped MLP projections
(gate and up W 11008x4096, down W 4096x11008, 2048 tokens, r=64, alpha=16).
One step = forward and backward (dX, dA, dB) of all three projections, with
inputs resident in HBM. Algorithmic FLOPs per projection are
4 M N K + 6 M r (K + N) (the frozen weight takes no gradient).

The same JSON line carries: the roofline of the dominant kernel (the fused
NF4 forward contraction) measured with HIP events around each launch; the
decode-shaped GEMV (W 4096x4096, M in {1,4,16}, r=16) as effective NF4
weight GB/s over 64 rotating weight stores (554 MB, more than twice the
256 MB last-level cache); quantization throughput; and the CPU oracle timed
on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("NF4 linear fwd+bwd TFLOP/s (large M); effective NF4 weight GB/s (M≤16)")
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t handles (libamdhip64) for timing single launches."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pool = []

    def pair(self):
        evs = []
        for _ in range(2):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            evs.append(e)
        self.pool.extend(evs)
        return tuple(evs)

    def ms(self, pair):
        self.hip.hipEventSynchronize(pair[1])
        out = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(out), pair[0], pair[1])
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(out.value)

    def close(self):
        for e in self.pool:
            self.hip.hipEventDestroy(e)
        self.pool = []


def run_prefill(args, q, synthetic, torch, dev, ev):
    M, r, alpha = 2048, 64, 16
    s = alpha / r
    projs = []
    wsb = 0
    for j, (N, K) in enumerate([(11008, 4096), (11008, 4096), (4096, 11008)]):
        W, X, A, B, dY = synthetic.linear_inputs(M, N, K, r, dev, seed=0,
                                                 base=synthetic.linear_base(0, j))
        st = q.qlora_nf4_quantize(W)
        p = dict(N=N, K=K, W=W, st=st, X=X, A=A, B=B, dY=dY,
                 Y=torch.empty(M, N, dtype=torch.bfloat16, device=dev),
                 T=torch.empty(M, r, dtype=torch.float32, device=dev),
                 dX=torch.empty(M, K, dtype=torch.bfloat16, device=dev),
                 dA=torch.empty(K, r, dtype=torch.float32, device=dev),
                 dB=torch.empty(r, N, dtype=torch.float32, device=dev))
        projs.append(p)
        wsb = max(wsb, q.qlora_linear_workspace_bytes(M, N, K, r))
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    flops_step = sum(4 * M * p["N"] * p["K"] + 6 * M * r * (p["K"] + p["N"]) for p in projs)
    fwd_kernel_flops = [2 * M * p["N"] * p["K"] + 2 * M * r * p["N"] for p in projs]
    dx_kernel_flops = [2 * M * p["N"] * p["K"] + 2 * M * r * p["K"] for p in projs]

    def step(events=None):
        for i, p in enumerate(projs):
            efwd = events[2 * i] if events else None
            ebwd = events[2 * i + 1] if events else None
            q.qlora_linear_fwd(p["X"], p["st"], p["A"], p["B"], s, Y=p["Y"], T=p["T"], ws=ws,
                               events=efwd)
            q.qlora_linear_bwd(p["dY"], p["X"], p["T"], p["st"], p["A"], p["B"], s, dX=p["dX"],
                               dA=p["dA"], dB=p["dB"], ws=ws, events=ebwd)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    kev = [[ev.pair() for _ in range(2 * len(projs))] for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for k in range(args.steps):
        step(kev[k])
    t1.record()
    torch.cuda.synchronize()
    ms_total = t0.elapsed_time(t1)
    ms_step = ms_total / args.steps
    fwd_ms = [[ev.ms(kev[k][2 * i]) for k in range(args.steps)] for i in range(len(projs))]
    dx_ms = [[ev.ms(kev[k][2 * i + 1]) for k in range(args.steps)] for i in range(len(projs))]
    fwd_avg = sum(sum(x) for x in fwd_ms) / (len(projs) * args.steps)
    dx_avg = sum(sum(x) for x in dx_ms) / (len(projs) * args.steps)
    fwd_flops_avg = sum(fwd_kernel_flops) / len(projs)
    dx_flops_avg = sum(dx_kernel_flops) / len(projs)
    res = dict(
        ms_per_step=ms_step,
        tflops=flops_step / (ms_step * 1e-3) / 1e12,
        flops_step=flops_step,
        fwd_kernel_ms=fwd_avg,
        fwd_kernel_tflops=fwd_flops_avg / (fwd_avg * 1e-3) / 1e12,
        fwd_kernel_flops=fwd_flops_avg,
        dx_kernel_ms=dx_avg,
        dx_kernel_tflops=dx_flops_avg / (dx_avg * 1e-3) / 1e12,
        per_proj_fwd_ms=[sum(x) / len(x) for x in fwd_ms],
        per_proj_dx_ms=[sum(x) / len(x) for x in dx_ms],
    )
    # quantization throughput on the gate weight (bf16 in, store out)
    W0 = projs[0]["W"]
    st0 = projs[0]["st"]
    qa, qb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        q.qlora_nf4_quantize(W0, out=st0)
    torch.cuda.synchronize()
    qa.record()
    for _ in range(10):
        q.qlora_nf4_quantize(W0, out=st0)
    qb.record()
    torch.cuda.synchronize()
    qms = qa.elapsed_time(qb) / 10
    res["quantize"] = dict(shape=[11008, 4096], ms=qms,
                           GBps=(2 * W0.numel() + st0.nbytes()) / (qms * 1e-3) / 1e9)
    return res, projs


def run_gemv(args, q, synthetic, torch, dev, ev):
    N = K = 4096
    r, alpha = 16, 32
    s = alpha / r
    nstores = args.gemv_stores
    stores = []
    for i in range(nstores):
        W = synthetic.normal((N, K), 0.02, dev, 100 + i, synthetic.W_IDX)
        stores.append(q.qlora_nf4_quantize(W))
        del W
    A = synthetic.normal((K, r), 0.01, dev, 0, synthetic.A_IDX)
    B = synthetic.normal((r, N), 0.01, dev, 0, synthetic.B_IDX)
    wbytes = stores[0].nbytes()
    out = {"weight_bytes_per_call": wbytes, "stores": nstores,
           "rotating_bytes": wbytes * nstores}
    for M in (1, 4, 16):
        X = synthetic.normal((M, K), 1.0, dev, 0, synthetic.X_IDX)
        Y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        T = torch.empty(M, r, dtype=torch.float32, device=dev)
        ws = torch.empty(q.qlora_linear_workspace_bytes(M, N, K, r), dtype=torch.uint8,
                         device=dev)
        for i in range(nstores):
            q.qlora_linear_fwd(X, stores[i], A, B, s, Y=Y, T=T, ws=ws)
        torch.cuda.synchronize()
        calls = nstores * args.gemv_rounds
        kev = [ev.pair() for _ in range(calls)]
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for c in range(calls):
            q.qlora_linear_fwd(X, stores[c % nstores], A, B, s, Y=Y, T=T, ws=ws, events=kev[c])
        t1.record()
        torch.cuda.synchronize()
        call_us = t0.elapsed_time(t1) * 1e3 / calls
        kern_us = sum(ev.ms(p) for p in kev) * 1e3 / calls
        gk = wbytes / (kern_us * 1e-6) / 1e9
        out[f"M{M}"] = dict(call_us=call_us, kernel_us=kern_us,
                            eff_weight_GBps_call=wbytes / (call_us * 1e-6) / 1e9,
                            eff_weight_GBps_kernel=gk,
                            roofline={"bound": "hbm", "achieved": round(gk, 1),
                                      "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                      "frac": round(gk / PEAK_HBM_GBPS, 4)})
        log(f"[gemv] M={M}: {call_us:.2f} us/call, kernel {kern_us:.2f} us, "
            f"{out[f'M{M}']['eff_weight_GBps_kernel']:.0f} GB/s (kernel)")
    del stores
    return out


def cpu_baseline(args, projs, torch):
    """The oracle, timed on this host on a bounded sample: forward and
    backward of the gate projection (11008x4096, r=64) for the first
    `cpu_rows` tokens, including its dequantization of the weight; the
    weight is quantized by the oracle before timing."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    p = projs[0]
    Mc = args.cpu_rows
    r = p["A"].shape[1]
    f = lambda t: t.detach().float().cpu().numpy()
    W = f(p["W"]).ravel()
    X, A, B, dY = f(p["X"][:Mc]), f(p["A"]), f(p["B"]), f(p["dY"][:Mc])
    ref = oracle.quantize(W)
    N, K = p["N"], p["K"]
    t0 = time.perf_counter()
    wp = oracle.dequantize(ref["codes"], ref["absmax_q"], ref["absmax_s2"], N * K).reshape(N, K)
    oracle.linear_fwd(X, wp, A, B, 0.25)
    oracle.linear_bwd(dY, X, wp, A, B, 0.25)
    dt = time.perf_counter() - t0
    flops = 4 * Mc * N * K + 6 * Mc * r * (K + N)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"gate projection 11008x4096, r=64, first {Mc} of 2048 tokens: "
                      f"dequantize + forward + backward in float64 numpy ({dt:.2f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--gemv-stores", type=int, default=64)
    ap.add_argument("--gemv-rounds", type=int, default=4)
    ap.add_argument("--cpu-rows", type=int, default=256)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-gemv", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not run "
              "(the data-parallel exchange of dA/dB is described in DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import bit_quantized_finetuning_quantize_amd as q
    import synthetic

    dev = torch.device("cuda:0")
    ev = HipEvents()
    log("[bench] prefill MLP fwd+bwd ...")
    pre, projs = run_prefill(args, q, synthetic, torch, dev, ev)
    log(f"[bench] {pre['tflops']:.1f} TFLOP/s, {pre['ms_per_step']:.3f} ms/step; fwd kernel "
        f"{pre['fwd_kernel_tflops']:.1f} TFLOP/s, dX kernel {pre['dx_kernel_tflops']:.1f}")
    gemv = None
    if not args.no_gemv:
        log("[bench] decode GEMV ...")
        gemv = run_gemv(args, q, synthetic, torch, dev, ev)
    cpu = None
    if not args.no_cpu:
        log("[bench] CPU oracle sample ...")
        cpu = cpu_baseline(args, projs, torch)
        log(f"[bench] cpu {cpu['value']:.4f} TFLOP/s")
    ev.close()

    line = {
        "metric": METRIC,
        "value": round(pre["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "prefill MLP projections: gate/up W 11008x4096 and down W 4096x11008 "
                        "NF4 (block 64, DQ 256), X 2048 tokens bf16, LoRA r=64 alpha=16, "
                        "fwd + bwd (dX, dA, dB) of all three per step",
            "tokens": 2048, "rank": 64, "alpha": 16,
            "flops_per_step": pre["flops_step"],
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "fused NF4 forward contraction (dequant + bf16 MFMA + LoRA segment)",
            "achieved": round(pre["fwd_kernel_tflops"], 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(pre["fwd_kernel_tflops"] / PEAK_BF16_TFLOPS, 4),
            "traffic": None,
            "flops_per_launch": pre["fwd_kernel_flops"],
            "avg_launch_ms": round(pre["fwd_kernel_ms"], 4),
        },
        "roofline_dx": {
            "bound": "mfma", "achieved": round(pre["dx_kernel_tflops"], 2),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(pre["dx_kernel_tflops"] / PEAK_BF16_TFLOPS, 4),
            "avg_launch_ms": round(pre["dx_kernel_ms"], 4),
        },
        "quantize": pre["quantize"],
        "gemv": gemv,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
