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


# HBM traffic of the forward contraction comes from two rocprofv3 --pmc runs
# of `bench.py --pmc-pass` (FETCH_SIZE, then WRITE_SIZE), each scaled by what
# the same counter reads for a plain elementwise kernel of known size, and
# is reported only while the kernel's sources are the ones it was taken on
# (one hash for the contractions' sources, one for the GEMV's).
PMC_FILE = os.path.join(ROOT, "profiles", "nf4_linear_traffic_pmc.json")
KERNEL_SOURCES = ["common.h", "gemm.h", "linear.hip"]
GEMV_SOURCES = ["common.h", "gemv.hip"]
CALIB_ELEMS = 64 << 20  # float32 in and out: 256 MiB read, 256 MiB written
PMC_SHAPE = dict(M=2048, N=11008, K=4096, r=64, alpha=16)
GEMV_PMC_SHAPE = dict(M=1, N=4096, K=4096, r=16, alpha=32, stores=64)


def kernel_source_hash(sources=KERNEL_SOURCES):
    """Hash of the kernel sources with comments and blank space removed, so
    that an edit of a comment leaves stored counter data valid."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "bit_quantized_finetuning_quantize_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def fwd_algorithmic_bytes(M, N, K, r, **_):
    """Bytes the forward contraction must move once: X, the NF4 store, the
    scaled adapter product s*T (bf16, rank padded to 64), B, and Y."""
    r64 = (r + 63) // 64 * 64
    nb = N * K // 64
    return (2 * M * K + N * K // 2 + nb + (nb + 255) // 256 * 4 + 2 * M * r64 + 2 * r * N
            + 2 * M * N)


def pmc_pass():
    """The dispatches the counter runs read: three calibration kernels, then
    three forward and three backward passes of the gate projection (the
    contractions are launches of each), then the decode GEMV (M = 1) once on
    each of 64 weight stores, so that every call reads its store from
    beyond the last-level cache."""
    import torch
    import bit_quantized_finetuning_quantize_amd as q
    import synthetic
    dev = torch.device("cuda:0")
    a = torch.ones(CALIB_ELEMS, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    for _ in range(3):
        torch.mul(a, 2.0, out=b)
    torch.cuda.synchronize()
    del a, b
    sh = PMC_SHAPE
    W, X, A, B, _ = synthetic.linear_inputs(sh["M"], sh["N"], sh["K"], sh["r"], dev, seed=0,
                                           base=synthetic.linear_base(0, 0))
    st = q.qlora_nf4_quantize(W)
    ws = q.workspace(sh["M"], sh["N"], sh["K"], sh["r"], dev)
    dY = synthetic.normal((sh["M"], sh["N"]), 1e-3, dev, 0, synthetic.DY_IDX)
    for _ in range(3):
        Y, T = q.qlora_linear_fwd(X, st, A, B, sh["alpha"] / sh["r"], ws=ws)
    for _ in range(3):
        q.qlora_linear_bwd(dY, X, T, st, A, B, sh["alpha"] / sh["r"], ws=ws)
    torch.cuda.synchronize()
    del W, X, A, B, st, ws, dY, Y, T
    g = GEMV_PMC_SHAPE
    stores = []
    for i in range(g["stores"]):
        Wg = synthetic.normal((g["N"], g["K"]), 0.02, dev, 100 + i, synthetic.W_IDX)
        stores.append(q.qlora_nf4_quantize(Wg))
        del Wg
    Ag = synthetic.normal((g["K"], g["r"]), 0.01, dev, 0, synthetic.A_IDX)
    Bg = synthetic.normal((g["r"], g["N"]), 0.01, dev, 0, synthetic.B_IDX)
    Xg = synthetic.normal((g["M"], g["K"]), 1.0, dev, 0, synthetic.X_IDX)
    Yg = torch.empty(g["M"], g["N"], dtype=torch.bfloat16, device=dev)
    wsg = torch.empty(q.qlora_linear_workspace_bytes(g["M"], g["N"], g["K"], g["r"]),
                      dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    for stg in stores:
        q.qlora_linear_fwd(Xg, stg, Ag, Bg, g["alpha"] / g["r"], want_T=False, Y=Yg, ws=wsg)
    torch.cuda.synchronize()
    log("[pmc] done")


def _pmc_values(d, counter):
    """Median counter value per dispatch of each kernel the pass launches:
    the calibration kernel, the forward and dX contractions, the GEMV."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    vals = {"calib": [], "fwd": [], "dx": [], "gemv": []}
    for fn in files:
        with open(fn) as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") != counter:
                    continue
                name = row.get("Kernel_Name", "")
                v = float(row["Counter_Value"])
                if "contraction_kernel" in name and "Nf4Rows" in name:
                    vals["fwd"].append(v)
                elif "contraction_kernel" in name and "Nf4Cols" in name:
                    vals["dx"].append(v)
                elif "nf4_gemv_kernel" in name:
                    vals["gemv"].append(v)
                elif "MulFunctor" in name and row.get("Grid_Size") == str(CALIB_ELEMS // 4):
                    vals["calib"].append(v)  # the calibration kernel: 4 floats per work-item
    for k, v in vals.items():
        if not v:
            raise SystemExit(f"{counter}: no {k} dispatches")
    med = lambda x: sorted(x)[len(x) // 2]
    return {k: (med(v), len(v)) for k, v in vals.items()}


def dx_algorithmic_bytes(M, N, K, r, **_):
    """Bytes the dX contraction must move once: dY, the NF4 store, s*G (bf16,
    rank padded to 64), the adapter A, and dX."""
    r64 = (r + 63) // 64 * 64
    nb = N * K // 64
    return (2 * M * N + N * K // 2 + nb + (nb + 255) // 256 * 4 + 2 * M * r64 + 2 * r * K
            + 2 * M * K)


def gemv_weight_bytes(N, K, **_):
    nb = N * K // 64
    return N * K // 2 + nb + (nb + 255) // 256 * 4


def pmc_summarize(fetch_dir, write_dir, cmd_fetch, cmd_write):
    vf = _pmc_values(fetch_dir, "FETCH_SIZE")
    vw = _pmc_values(write_dir, "WRITE_SIZE")
    calib_bytes = 4 * CALIB_ELEMS
    k_fetch = vf["calib"][0] * 1024 / calib_bytes   # counter bytes per true byte
    k_write = vw["calib"][0] * 1024 / calib_bytes

    def entry(key, alg):
        fetch = vf[key][0] * 1024 / k_fetch
        write = vw[key][0] * 1024 / k_write
        e = {"FETCH_SIZE_KiB": vf[key][0], "WRITE_SIZE_KiB": vw[key][0],
             "dispatches": [vf[key][1], vw[key][1]],
             "fetch_bytes": round(fetch), "write_bytes": round(write),
             "traffic_bytes": round(fetch + write)}
        if alg:
            e["algorithmic_bytes"] = alg
            e["traffic_over_algorithmic"] = round((fetch + write) / alg, 3)
        return e

    g = GEMV_PMC_SHAPE
    out = {
        "kernel": "contraction_kernel (NF4 forward: DirectRows<256>, Nf4Rows<128> + LoRA segment)",
        "workload": "gate projection W 11008x4096 NF4, X 2048x4096 bf16, r=64",
        "source_hash": kernel_source_hash(),
        "sources": KERNEL_SOURCES,
        "gemv_source_hash": kernel_source_hash(GEMV_SOURCES),
        "gemv_sources": GEMV_SOURCES,
        "calibration": {"kernel": "torch.mul(float32[64Mi], 2.0, out=float32[64Mi])",
                        "bytes_read": calib_bytes, "bytes_written": calib_bytes,
                        "FETCH_SIZE_KiB": vf["calib"][0], "WRITE_SIZE_KiB": vw["calib"][0],
                        "fetch_factor": round(k_fetch, 4), "write_factor": round(k_write, 4),
                        "dispatches": [vf["calib"][1], vw["calib"][1]]},
        "forward": entry("fwd", fwd_algorithmic_bytes(**PMC_SHAPE)),
        "dx": entry("dx", dx_algorithmic_bytes(**PMC_SHAPE)),
        "gemv": dict(entry("gemv", None), workload="decode GEMV W 4096x4096 NF4, M=1, r=16, "
                     "one call (one launch) on each of 64 stores",
                     weight_bytes=gemv_weight_bytes(**g)),
        "commands": [cmd_fetch, cmd_write],
    }
    os.makedirs(os.path.dirname(PMC_FILE), exist_ok=True)
    with open(PMC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def stored_counters(gemv=False):
    """The stored counter summary, or (None, why) when there is none or the
    sources of the contractions (gemv=False) or of the GEMV (gemv=True)
    changed since it was taken."""
    try:
        with open(PMC_FILE) as fh:
            d = json.load(fh)
    except (OSError, ValueError):
        return None, "no counter summary"
    key, src = ("gemv_source_hash", GEMV_SOURCES) if gemv else ("source_hash", KERNEL_SOURCES)
    if d.get(key) != kernel_source_hash(src):
        return None, "kernel changed since the counters were taken"
    return d, None


def stored_traffic():
    """(bytes per launch, detail) of the forward contraction, or (None, why)."""
    d, why = stored_counters()
    if d is None:
        return None, why
    f = d["forward"]
    return f["traffic_bytes"], {"fetch_bytes": f["fetch_bytes"], "write_bytes": f["write_bytes"],
                                "algorithmic_bytes": f["algorithmic_bytes"],
                                "from": os.path.relpath(PMC_FILE, ROOT)}


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
    # timed region: the steps alone (the per-kernel events of the second
    # pass put idle time between launches, so they stay outside it)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for k in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms_total = t0.elapsed_time(t1)
    ms_step = ms_total / args.steps
    # second pass: HIP events on the launch stream around each main kernel
    kev = [[ev.pair() for _ in range(2 * len(projs))] for _ in range(args.steps)]
    for k in range(args.steps):
        step(kev[k])
    torch.cuda.synchronize()
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
    # One launch moves 113 MB in about 25 us, less than the host needs to
    # issue a call, so back-to-back calls from Python would time the host:
    # 10 launches are captured once into a HIP graph and the replays timed.
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            q.qlora_nf4_quantize(W0, out=st0)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(10):
            q.qlora_nf4_quantize(W0, out=st0)
    graph.replay()
    torch.cuda.synchronize()
    qms = float("inf")
    for _ in range(5):
        qa.record()
        graph.replay()
        qb.record()
        torch.cuda.synchronize()
        qms = min(qms, qa.elapsed_time(qb) / 10)
    del graph
    qbytes = 2 * W0.numel() + st0.nbytes()
    res["quantize"] = dict(shape=[11008, 4096], ms=qms, bytes=qbytes,
                           GBps=qbytes / (qms * 1e-3) / 1e9,
                           frac_of_hbm_peak=qbytes / (qms * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                           what="10 launches replayed from a HIP graph, best of 5 replays")
    # standalone dequantization of the same store, float32 and bf16 out
    w32 = torch.empty(W0.numel(), dtype=torch.float32, device=dev)
    w16 = torch.empty(W0.numel(), dtype=torch.bfloat16, device=dev)
    deq = {}
    for name, fn, outb, bpe in (("f32", q.qlora_nf4_dequantize, w32, 4),
                                ("bf16", q.qlora_nf4_dequantize_bf16, w16, 2)):
        for _ in range(3):
            fn(st0, out=outb)
        torch.cuda.synchronize()
        qa.record()
        for _ in range(10):
            fn(st0, out=outb)
        qb.record()
        torch.cuda.synchronize()
        dms = qa.elapsed_time(qb) / 10
        deq[name] = dict(ms=dms, GBps=(st0.nbytes() + bpe * W0.numel()) / (dms * 1e-3) / 1e9)
    res["dequantize"] = dict(shape=[11008, 4096], **deq)
    del w32, w16
    # adapter merge into a bf16 copy of the same weight (store in, bf16 out)
    A0, B0 = projs[0]["A"], projs[0]["B"]
    merged = q.qlora_nf4_merge(st0, A0, B0, s)
    for _ in range(2):
        q.qlora_nf4_merge(st0, A0, B0, s, out=merged)
    torch.cuda.synchronize()
    qa.record()
    for _ in range(10):
        q.qlora_nf4_merge(st0, A0, B0, s, out=merged)
    qb.record()
    torch.cuda.synchronize()
    mms = qa.elapsed_time(qb) / 10
    # AdamW step over every adapter of the 32-layer 7B-style stack at r = 64
    na = 32 * r * (4 * (4096 + 4096) + 2 * (4096 + 11008) + (11008 + 4096))
    st_p, st_m, st_v, st_g = (torch.zeros(na, dtype=torch.float32, device=dev) for _ in range(4))
    st_16 = torch.empty(na, dtype=torch.bfloat16, device=dev)
    for t in range(1, 3):
        q.qlora_adamw_step(st_p, st_m, st_v, st_g, 2e-4, step=t, weight_decay=0.01, p_bf16=st_16)
    torch.cuda.synchronize()
    qa.record()
    for t in range(3, 8):
        q.qlora_adamw_step(st_p, st_m, st_v, st_g, 2e-4, step=t, weight_decay=0.01, p_bf16=st_16)
    qb.record()
    torch.cuda.synchronize()
    ams = qa.elapsed_time(qb) / 5
    res["adamw"] = dict(params=na, ms=ams, bytes_per_param=30,
                        GBps=30 * na / (ams * 1e-3) / 1e9)
    del st_m, st_v
    # the same step with 8-bit moments (codes and per-256 scales); a random
    # gradient, so that every block encodes non-zero moments
    st_g.normal_(0.0, 1e-3)
    m8, sm8, v8, sv8 = q.adamw8_state(na, dev)
    for t in range(1, 3):
        q.qlora_adamw8_step(st_p, m8, sm8, v8, sv8, st_g, 2e-4, step=t, weight_decay=0.01,
                            p_bf16=st_16)
    torch.cuda.synchronize()
    qa.record()
    for t in range(3, 8):
        q.qlora_adamw8_step(st_p, m8, sm8, v8, sv8, st_g, 2e-4, step=t, weight_decay=0.01,
                            p_bf16=st_16)
    qb.record()
    torch.cuda.synchronize()
    a8ms = qa.elapsed_time(qb) / 5
    b8 = 18 + 16 / 256  # p, g, codes in and out, bf16 p, scales
    res["adamw8"] = dict(params=na, ms=a8ms, bytes_per_param=round(b8, 4),
                         GBps=b8 * na / (a8ms * 1e-3) / 1e9,
                         state_bytes=2 * na + 8 * ((na + 255) // 256))
    del m8, sm8, v8, sv8
    # the same two steps with the optimizer state in pinned host memory
    # (hipHostMalloc, mapped): the moments cross the host link on every step
    host = {}
    for name in ("adamw_host", "adamw8_host"):
        if name == "adamw_host":
            hm, hv = q.adamw_state(na, dev, host=True)
            fn = lambda t: q.qlora_adamw_step(st_p, hm, hv, st_g, 2e-4, step=t, weight_decay=0.01,
                                              p_bf16=st_16)
            state_bytes = 8 * na  # m and v, read and written
        else:
            hm8, hsm8, hv8, hsv8 = q.adamw8_state(na, dev, host=True)
            fn = lambda t: q.qlora_adamw8_step(st_p, hm8, hsm8, hv8, hsv8, st_g, 2e-4, step=t,
                                               weight_decay=0.01, p_bf16=st_16)
            state_bytes = 2 * na + 8 * ((na + 255) // 256)
        fn(1)
        torch.cuda.synchronize()
        qa.record()
        for t in range(2, 5):
            fn(t)
        qb.record()
        torch.cuda.synchronize()
        hms = qa.elapsed_time(qb) / 3
        host[name] = dict(params=na, ms=hms, state_bytes=state_bytes,
                          host_link_GBps=2 * state_bytes / (hms * 1e-3) / 1e9,
                          what="moments in pinned host memory, read and written in place")
        log(f"[bench] {name}: {hms:.2f} ms per step")
    res.update(host)
    del st_p, st_g, st_16
    res["merge"] = dict(shape=[11008, 4096], rank=r, ms=mms,
                        GBps=(st0.nbytes() + 2 * W0.numel()) / (mms * 1e-3) / 1e9,
                        rank_flops_TFLOPs=2 * W0.numel() * r / (mms * 1e-3) / 1e12)
    # the same step with LoRA dropout p = 0.05 on every adapter input: one
    # keep mask drawn per projection and step, fwd and bwd through it
    pd = 0.05
    masks = [torch.empty(M, pr["K"] // 32, dtype=torch.int32, device=dev) for pr in projs]

    def dstep(it):
        for i, pr in enumerate(projs):
            q.qlora_dropout_mask(M, pr["K"], pd, 1234 + i, it, out=masks[i])
            q.qlora_linear_fwd_dropout(pr["X"], pr["st"], pr["A"], pr["B"], s, masks[i], pd,
                                       Y=pr["Y"], T=pr["T"], ws=ws)
            q.qlora_linear_bwd_dropout(pr["dY"], pr["X"], pr["T"], pr["st"], pr["A"], pr["B"], s,
                                       masks[i], pd, dX=pr["dX"], dA=pr["dA"], dB=pr["dB"],
                                       ws=ws)

    for it in range(args.warmup):
        dstep(it)
    torch.cuda.synchronize()
    qa.record()
    for it in range(args.steps):
        dstep(args.warmup + it)
    qb.record()
    torch.cuda.synchronize()
    dms = qa.elapsed_time(qb) / args.steps
    mk = masks[2]  # the down projection's input, 2048 x 11008
    for _ in range(2):
        q.qlora_dropout_mask(M, 11008, pd, 1, 0, out=mk)
    torch.cuda.synchronize()
    qa.record()
    for it in range(10):
        q.qlora_dropout_mask(M, 11008, pd, 1, it, out=mk)
    qb.record()
    torch.cuda.synchronize()
    mkms = qa.elapsed_time(qb) / 10
    # context: the step's two weight products done the unfused way, per
    # projection a bf16 dequantization of the store and a vendor bf16 GEMM
    # (torch.matmul on two 2-D tensors: hipBLASLt), for Y and again for dX
    w16 = torch.empty(max(pr["N"] * pr["K"] for pr in projs), dtype=torch.bfloat16, device=dev)

    def unfused():
        for pr in projs:
            W16 = q.qlora_nf4_dequantize_bf16(pr["st"], out=w16[:pr["N"] * pr["K"]])
            W16 = W16.view(pr["N"], pr["K"])
            torch.matmul(pr["X"], W16.t(), out=pr["Y"])
            W16 = q.qlora_nf4_dequantize_bf16(pr["st"], out=w16[:pr["N"] * pr["K"]])
            W16 = W16.view(pr["N"], pr["K"])
            torch.matmul(pr["dY"], W16, out=pr["dX"])

    for _ in range(args.warmup):
        unfused()
    torch.cuda.synchronize()
    qa.record()
    for _ in range(args.steps):
        unfused()
    qb.record()
    torch.cuda.synchronize()
    ums = qa.elapsed_time(qb) / args.steps
    # the vendor GEMM alone per projection (forward, then dX), 10 calls each
    gemm_ms = []
    for pr in projs:
        W16 = q.qlora_nf4_dequantize_bf16(pr["st"], out=w16[:pr["N"] * pr["K"]])
        W16 = W16.view(pr["N"], pr["K"])
        pair = []
        for fn in (lambda: torch.matmul(pr["X"], W16.t(), out=pr["Y"]),
                   lambda: torch.matmul(pr["dY"], W16, out=pr["dX"])):
            fn()
            torch.cuda.synchronize()
            qa.record()
            for _ in range(10):
                fn()
            qb.record()
            torch.cuda.synchronize()
            pair.append(round(qa.elapsed_time(qb) / 10, 4))
        gemm_ms.append(pair)
    res["unfused_reference"] = dict(
        ms=ums, fused_ms=sum(res["per_proj_fwd_ms"]) + sum(res["per_proj_dx_ms"]),
        vendor_gemm_ms_fwd_dx=gemm_ms,
        what="per projection: qlora_nf4_dequantize_bf16 + torch.matmul (hipBLASLt) for Y, and "
             "again for dX; against the fused forward and dX kernels of the same step")
    del w16
    # the plain step on stores without double quantization
    nodq = [q.qlora_nf4_quantize(pr["W"], double_quant=False) for pr in projs]

    def nstep():
        for pr, st in zip(projs, nodq):
            q.qlora_linear_fwd(pr["X"], st, pr["A"], pr["B"], s, Y=pr["Y"], T=pr["T"], ws=ws)
            q.qlora_linear_bwd(pr["dY"], pr["X"], pr["T"], st, pr["A"], pr["B"], s, dX=pr["dX"],
                               dA=pr["dA"], dB=pr["dB"], ws=ws)

    for _ in range(args.warmup):
        nstep()
    torch.cuda.synchronize()
    qa.record()
    for _ in range(args.steps):
        nstep()
    qb.record()
    torch.cuda.synchronize()
    nms = qa.elapsed_time(qb) / args.steps
    res["nodq"] = dict(ms_per_step=nms, tflops=flops_step / (nms * 1e-3) / 1e12,
                       store_bytes=sum(st.nbytes() for st in nodq),
                       dq_store_bytes=sum(pr["st"].nbytes() for pr in projs))
    del nodq
    res["dropout"] = dict(p=pd, ms_per_step=dms, tflops=flops_step / (dms * 1e-3) / 1e12,
                          mask_shape=[M, 11008], mask_ms=mkms,
                          mask_Gelem_per_s=M * 11008 / (mkms * 1e-3) / 1e9)
    del masks
    return res, projs


def run_gemv(args, q, synthetic, torch, dev):
    """Decode GEMV per call, timed by replaying a HIP graph of `nstores`
    back-to-back calls (each on a different weight store), so that host
    launch overhead is not counted; a call is one launch."""
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
           "rotating_bytes": wbytes * nstores, "timing": "HIP graph replay of back-to-back calls"}
    def call_time(M, stores):
        X = synthetic.normal((M, K), 1.0, dev, 0, synthetic.X_IDX)
        Y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        ws = torch.empty(q.qlora_linear_workspace_bytes(M, N, K, r), dtype=torch.uint8,
                         device=dev)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(nstores):
                q.qlora_linear_fwd(X, stores[i], A, B, s, want_T=False, Y=Y, ws=ws)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(nstores):
                q.qlora_linear_fwd(X, stores[i], A, B, s, want_T=False, Y=Y, ws=ws)
        g.replay()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(args.gemv_rounds):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) * 1e3 / (args.gemv_rounds * nstores)

    for M in (1, 4, 16):
        call_us = call_time(M, stores)
        gbps = wbytes / (call_us * 1e-6) / 1e9
        # every byte a call must move once: the store, X, A, B and Y
        tbytes = wbytes + 2 * (M * K + K * r + r * N + M * N)
        out[f"M{M}"] = dict(call_us=round(call_us, 3), eff_weight_GBps=round(gbps, 1),
                            total_bytes=tbytes,
                            total_GBps=round(tbytes / (call_us * 1e-6) / 1e9, 1),
                            roofline={"bound": "hbm", "achieved": round(gbps, 1),
                                      "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                      "frac": round(gbps / PEAK_HBM_GBPS, 4),
                                      "per": "call (one launch: the T = X A workgroups and the "
                                              "row-tile workgroups)"})
        log(f"[gemv] M={M}: {call_us:.2f} us/call, {gbps:.0f} GB/s effective weight")
    # context for the per-call figures: one vectorized torch elementwise
    # launch that reads the same number of bytes (an int64 view, compared
    # with 0: one byte written per eight read) from 64 rotating buffers, in
    # the same graph replay -- about the floor of a launch that streams a
    # store of this size from HBM
    bufs = [torch.zeros(wbytes // 8, dtype=torch.int64, device=dev) for _ in range(nstores)]
    flags = torch.empty(wbytes // 8, dtype=torch.bool, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for b in bufs:
            torch.ne(b, 0, out=flags)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    gs = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gs):
        for b in bufs:
            torch.ne(b, 0, out=flags)
    gs.replay()
    torch.cuda.synchronize()
    ta = torch.cuda.Event(enable_timing=True)
    tb = torch.cuda.Event(enable_timing=True)
    ta.record()
    for _ in range(args.gemv_rounds):
        gs.replay()
    tb.record()
    torch.cuda.synchronize()
    sus = ta.elapsed_time(tb) * 1e3 / (args.gemv_rounds * nstores)
    sb = (wbytes // 8) * 8
    out["stream_floor"] = dict(call_us=round(sus, 3), bytes_read=sb, bytes_written=sb // 8,
                               GBps=round(sb / (sus * 1e-6) / 1e9, 1),
                               what="torch.ne(int64 view, 0) over the store's bytes, "
                                    "64 rotating buffers, HIP-graph replay")
    log(f"[gemv] streaming floor (torch.ne over {sb} B): {sus:.2f} us per launch")
    # each call's time against that of the launch that only streams its bytes
    for M in (1, 4, 16):
        out[f"M{M}"]["frac_of_stream_floor"] = round(sus / out[f"M{M}"]["call_us"], 4)
    del gs, bufs, flags
    # the same calls on stores without double quantization (float32 block
    # constants, 4.5 bits per weight)
    del stores
    stores = []
    for i in range(nstores):
        W = synthetic.normal((N, K), 0.02, dev, 100 + i, synthetic.W_IDX)
        stores.append(q.qlora_nf4_quantize(W, double_quant=False))
        del W
    nb = stores[0].nbytes()
    us1 = call_time(1, stores)
    out["nodq_M1"] = dict(call_us=round(us1, 3), weight_bytes_per_call=nb,
                          eff_weight_GBps=round(nb / (us1 * 1e-6) / 1e9, 1))
    log(f"[gemv] no double quantization, M=1: {us1:.2f} us/call")
    del stores
    return out


def run_single(args, q, synthetic, torch, dev):
    """The single small linear (W 256x256 NF4, 16 tokens, r=8, alpha=16):
    quantize, forward and backward (dX, dA, dB), timed by replaying a HIP
    graph of 64 back-to-back sequences (every launch of the three calls
    inside). Launch-bound at this size: reported, not a throughput target."""
    M, N, K, r, alpha = 16, 256, 256, 8, 16
    s = alpha / r
    W, X, A, B, dY = synthetic.linear_inputs(M, N, K, r, dev, seed=0)
    st = q.qlora_nf4_quantize(W)
    ws = q.workspace(M, N, K, r, dev)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    T = torch.empty(M, r, dtype=torch.float32, device=dev)
    dX = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
    dA = torch.empty(K, r, dtype=torch.float32, device=dev)
    dB = torch.empty(r, N, dtype=torch.float32, device=dev)
    reps = 64

    def seq():
        q.qlora_nf4_quantize(W, out=st)
        q.qlora_linear_fwd(X, st, A, B, s, Y=Y, T=T, ws=ws)
        q.qlora_linear_bwd(dY, X, T, st, A, B, s, dX=dX, dA=dA, dB=dB, ws=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        seq()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            seq()
    g.replay()
    torch.cuda.synchronize()
    best = None
    for _ in range(3):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        g.replay()
        t1.record()
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) * 1e3 / reps
        best = us if best is None else min(best, us)
    flops = 4 * M * N * K + 6 * M * r * (K + N)
    out = dict(workload="single linear W 256x256 NF4 (block 64, DQ 256), X 16x256, r=8 "
                        "alpha=16: quantize + fwd + bwd (dX, dA, dB)",
               us_per_sequence=round(best, 3), flops=flops,
               timing="HIP graph replay of 64 back-to-back sequences, best of 3")
    log(f"[single] 256x256, 16 tokens: {best:.2f} us per quantize + fwd + bwd")
    del g
    return out


def run_stack7b(args, q, synthetic, torch, dev):
    """The 7B-style decoder stack: 32 layers x (q, k, v, o 4096x4096; gate, up
    11008x4096; down 4096x11008), N(0, 0.02) weights quantized to NF4 and kept
    resident (3,340,771,328 bytes), LoRA r=64 alpha=16 on every linear, 2048
    tokens. One sweep: the forward of every linear from layer 0 to layer 31,
    then the backward (dX, dA, dB) from layer 31 back to layer 0, so each
    store streams from HBM twice per sweep. Each linear type draws its own
    activations (the same for every layer: an activation feeding a layer has
    just been written, so it is cache-resident either way); the weights,
    adapters and outputs are per layer."""
    M, r, alpha = 2048, 64, 16
    s = alpha / r
    shapes = synthetic.LLAMA7B
    acts = []
    for j, (N, K) in enumerate(shapes):
        base = synthetic.linear_base(0, j)
        acts.append(dict(X=synthetic.normal((M, K), 1.0, dev, 0, base + synthetic.X_IDX),
                         dY=synthetic.normal((M, N), 1e-3, dev, 0, base + synthetic.DY_IDX)))
    lin = []
    for layer in range(32):
        for j, (N, K) in enumerate(shapes):
            base = synthetic.linear_base(layer, j)
            W = synthetic.normal((N, K), 0.02, dev, 0, base + synthetic.W_IDX)
            st = q.qlora_nf4_quantize(W)
            del W
            lin.append(dict(N=N, K=K, j=j, st=st,
                            A=synthetic.normal((K, r), 0.01, dev, 0, base + synthetic.A_IDX),
                            B=synthetic.normal((r, N), 0.01, dev, 0, base + synthetic.B_IDX),
                            T=torch.empty(M, r, dtype=torch.float32, device=dev),
                            dA=torch.empty(K, r, dtype=torch.float32, device=dev),
                            dB=torch.empty(r, N, dtype=torch.float32, device=dev)))
    store_bytes = sum(L["st"].nbytes() for L in lin)
    Ybuf = {n: torch.empty(M, n, dtype=torch.bfloat16, device=dev) for n in (4096, 11008)}
    dXbuf = {k: torch.empty(M, k, dtype=torch.bfloat16, device=dev) for k in (4096, 11008)}
    ws = q.workspace(M, 11008, 11008, r, dev)
    flops = sum(4 * M * L["N"] * L["K"] + 6 * M * r * (L["K"] + L["N"]) for L in lin)

    def sweep():
        for L in lin:
            a = acts[L["j"]]
            q.qlora_linear_fwd(a["X"], L["st"], L["A"], L["B"], s, Y=Ybuf[L["N"]], T=L["T"], ws=ws)
        for L in reversed(lin):
            a = acts[L["j"]]
            q.qlora_linear_bwd(a["dY"], a["X"], L["T"], L["st"], L["A"], L["B"], s,
                               dX=dXbuf[L["K"]], dA=L["dA"], dB=L["dB"], ws=ws)

    sweep()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.stack_sweeps):
        sweep()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.stack_sweeps
    out = dict(workload="32 layers x 7 linears (4096x4096 x4, 11008x4096 x2, 4096x11008), "
                        "2048 tokens, r=64: forward L0..L31 then backward L31..L0",
               ms_per_sweep=round(ms, 3), flops_per_sweep=flops,
               tflops=round(flops / (ms * 1e-3) / 1e12, 2),
               frac_of_bf16_peak=round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
               store_bytes=store_bytes, sweeps=args.stack_sweeps)
    log(f"[bench] 7B-style sweep: {ms:.2f} ms, {out['tflops']} TFLOP/s")
    del lin, acts, Ybuf, dXbuf, ws
    torch.cuda.empty_cache()
    return out


def run_stress65b(args, q, synthetic, torch, dev):
    """The 65B-shaped stack: all 560 Student-t(5) x 0.02 weights of 80 layers
    x (q, k, v, o 8192x8192; gate, up 22016x8192; down 8192x22016) quantized
    on the device and kept resident (33,407,713,280 bytes); the quantization
    kernels are timed alone (each layer's weights drawn first, then its
    seven quantizations into stores allocated beforehand between two
    events). Then layer 0 forward and
    backward at 4096 tokens (4 x 1024), r=64 alpha=16."""
    shapes = synthetic.LLAMA65B
    stores = []
    qms, nel = 0.0, 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for layer in range(80):
        Ws = [synthetic.student_t((N, K), 5, 0.02, dev, 0,
                                  synthetic.linear_base(layer, j) + synthetic.W_IDX)
              for j, (N, K) in enumerate(shapes)]
        outs = [q.empty_store(W.numel(), dev, W.shape) for W in Ws]
        torch.cuda.synchronize()
        e0.record()
        for W, st in zip(Ws, outs):
            stores.append(q.qlora_nf4_quantize(W, out=st))
        e1.record()
        torch.cuda.synchronize()
        qms += e0.elapsed_time(e1)
        nel += sum(W.numel() for W in Ws)
        del Ws
    store_bytes = sum(st.nbytes() for st in stores)
    quant = dict(weights=len(stores), params=nel, store_bytes=store_bytes, ms=round(qms, 3),
                 GBps=round((2 * nel + store_bytes) / (qms * 1e-3) / 1e9, 1),
                 what="bf16 read + NF4 store written, stores allocated first, kernels "
                      "between events per layer")
    log(f"[bench] 65B-shaped quantize all: {qms:.1f} ms, {quant['GBps']} GB/s, "
        f"{store_bytes} B resident")
    M, r, alpha = 4096, 64, 16
    s = alpha / r
    lay = []
    for j, (N, K) in enumerate(shapes):
        base = synthetic.linear_base(0, j)
        lay.append(dict(N=N, K=K, st=stores[j],
                        X=synthetic.normal((M, K), 1.0, dev, 0, base + synthetic.X_IDX),
                        dY=synthetic.normal((M, N), 1e-3, dev, 0, base + synthetic.DY_IDX),
                        A=synthetic.normal((K, r), 0.01, dev, 0, base + synthetic.A_IDX),
                        B=synthetic.normal((r, N), 0.01, dev, 0, base + synthetic.B_IDX),
                        Y=torch.empty(M, N, dtype=torch.bfloat16, device=dev),
                        T=torch.empty(M, r, dtype=torch.float32, device=dev),
                        dX=torch.empty(M, K, dtype=torch.bfloat16, device=dev),
                        dA=torch.empty(K, r, dtype=torch.float32, device=dev),
                        dB=torch.empty(r, N, dtype=torch.float32, device=dev)))
    ws = q.workspace(M, 22016, 22016, r, dev)
    flops = sum(4 * M * L["N"] * L["K"] + 6 * M * r * (L["K"] + L["N"]) for L in lay)

    def layer_step():
        for L in lay:
            q.qlora_linear_fwd(L["X"], L["st"], L["A"], L["B"], s, Y=L["Y"], T=L["T"], ws=ws)
        for L in reversed(lay):
            q.qlora_linear_bwd(L["dY"], L["X"], L["T"], L["st"], L["A"], L["B"], s, dX=L["dX"],
                               dA=L["dA"], dB=L["dB"], ws=ws)

    layer_step()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.stack_sweeps):
        layer_step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.stack_sweeps
    one = dict(workload="layer 0 of the 65B-shaped stack (8192x8192 x4, 22016x8192 x2, "
                        "8192x22016), 4096 tokens, r=64, fwd + bwd, the other 79 layers' "
                        "stores resident",
               ms=round(ms, 3), flops=flops, tflops=round(flops / (ms * 1e-3) / 1e12, 2),
               frac_of_bf16_peak=round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4))
    log(f"[bench] 65B-shaped layer fwd+bwd at 4096 tokens: {ms:.2f} ms, {one['tflops']} TFLOP/s")
    del lay, stores, ws
    torch.cuda.empty_cache()
    return dict(quantize_all=quant, layer=one)


def cpu_baseline(args, projs, torch):
    """The oracle, timed on this host on a bounded sample: forward and
    backward of the three projections, r=64, for the first `cpu_rows` tokens
    each, `cpu_reps` times, including the dequantization of each weight; the
    weights are quantized by the oracle before timing."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    Mc = args.cpu_rows
    f = lambda t: t.detach().float().cpu().numpy()
    prepared = []
    for p in projs:
        W = f(p["W"]).ravel()
        prepared.append((p, oracle.quantize(W), f(p["X"][:Mc]), f(p["A"]), f(p["B"]),
                         f(p["dY"][:Mc])))
    flops, dt = 0, 0.0
    for _ in range(args.cpu_reps):
        for p, ref, X, A, B, dY in prepared:
            r = A.shape[1]
            N, K = p["N"], p["K"]
            t0 = time.perf_counter()
            wp = oracle.dequantize(ref["codes"], ref["absmax_q"], ref["absmax_s2"],
                                   N * K).reshape(N, K)
            oracle.linear_fwd(X, wp, A, B, 0.25)
            oracle.linear_bwd(dY, X, wp, A, B, 0.25)
            dt += time.perf_counter() - t0
            flops += 4 * Mc * N * K + 6 * Mc * r * (K + N)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"the three projections (gate, up, down), r=64, first {Mc} of 2048 tokens "
                      f"each, {args.cpu_reps} times: dequantize + forward + backward in float64 "
                      f"numpy ({dt:.2f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--gemv-stores", type=int, default=64)
    ap.add_argument("--gemv-rounds", type=int, default=8)
    ap.add_argument("--cpu-rows", type=int, default=2048)
    ap.add_argument("--cpu-reps", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-gemv", action="store_true")
    ap.add_argument("--no-stacks", action="store_true",
                    help="skip the 7B-style sweep and the 65B-shaped legs")
    ap.add_argument("--only-stacks", action="store_true",
                    help="run only the 7B-style sweep and the 65B-shaped legs")
    ap.add_argument("--stack-sweeps", type=int, default=3)
    ap.add_argument("--pmc-pass", action="store_true",
                    help="run only the dispatches the counter runs read")
    ap.add_argument("--pmc-summarize", nargs=4,
                    metavar=("FETCH_DIR", "WRITE_DIR", "FETCH_CMD", "WRITE_CMD"),
                    help="turn two rocprofv3 --pmc outputs into the stored traffic summary")
    args = ap.parse_args()
    if args.pmc_summarize:
        pmc_summarize(*args.pmc_summarize)
        return
    if args.gpus != 1:
        print(f"bench.py: only one GPU is measured; --gpus {args.gpus} is not run",
              file=sys.stderr)
        sys.exit(2)

    if args.pmc_pass:
        pmc_pass()
        return

    import torch
    import bit_quantized_finetuning_quantize_amd as q
    import synthetic

    dev = torch.device("cuda:0")
    if args.only_stacks:
        print(json.dumps({"stack_7b": run_stack7b(args, q, synthetic, torch, dev),
                          "stress_65b": run_stress65b(args, q, synthetic, torch, dev)}), flush=True)
        return
    ev = HipEvents()
    log("[bench] prefill MLP fwd+bwd ...")
    pre, projs = run_prefill(args, q, synthetic, torch, dev, ev)
    log(f"[bench] {pre['tflops']:.1f} TFLOP/s, {pre['ms_per_step']:.3f} ms/step; fwd kernel "
        f"{pre['fwd_kernel_tflops']:.1f} TFLOP/s, dX kernel {pre['dx_kernel_tflops']:.1f}")
    gemv = None
    single = None
    if not args.no_gemv:
        log("[bench] decode GEMV ...")
        gemv = run_gemv(args, q, synthetic, torch, dev)
        log("[bench] single small linear ...")
        single = run_single(args, q, synthetic, torch, dev)
    stacks = None
    if not args.no_stacks:
        log("[bench] 7B-style stack sweep and 65B-shaped legs ...")
        stacks = {"stack_7b": run_stack7b(args, q, synthetic, torch, dev),
                  "stress_65b": run_stress65b(args, q, synthetic, torch, dev)}
    cpu = None
    if not args.no_cpu:
        log("[bench] CPU oracle sample ...")
        cpu = cpu_baseline(args, projs, torch)
        log(f"[bench] cpu {cpu['value']:.4f} TFLOP/s")
    ev.close()
    traffic, traffic_detail = stored_traffic()
    counters, _ = stored_counters()
    dx_traffic = counters["dx"]["traffic_bytes"] if counters and "dx" in counters else None
    gcounters, _ = stored_counters(gemv=True)
    if gemv is not None and gcounters and "gemv" in gcounters:
        # HBM bytes of a call's one launch
        gemv["M1"]["roofline"]["traffic"] = gcounters["gemv"]["traffic_bytes"]

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
            "traffic": traffic,
            "traffic_detail": traffic_detail,
            "flops_per_launch": pre["fwd_kernel_flops"],
            "avg_launch_ms": round(pre["fwd_kernel_ms"], 4),
        },
        "roofline_dx": {
            "bound": "mfma", "achieved": round(pre["dx_kernel_tflops"], 2),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(pre["dx_kernel_tflops"] / PEAK_BF16_TFLOPS, 4),
            "avg_launch_ms": round(pre["dx_kernel_ms"], 4),
            "traffic": dx_traffic,
        },
        "prefill_kernels_ms": {"fwd": [round(x, 4) for x in pre["per_proj_fwd_ms"]],
                               "dx": [round(x, 4) for x in pre["per_proj_dx_ms"]],
                               "order": ["gate 11008x4096", "up 11008x4096",
                                         "down 4096x11008"]},
        "unfused_reference": pre["unfused_reference"],
        "quantize": pre["quantize"],
        "dequantize": pre["dequantize"],
        "merge": pre["merge"],
        "adamw": pre["adamw"],
        "adamw8": pre["adamw8"],
        "adamw_host": pre["adamw_host"],
        "adamw8_host": pre["adamw8_host"],
        "dropout": pre["dropout"],
        "nodq": pre["nodq"],
        "gemv": gemv,
        "single_linear": single,
        "stacks": stacks,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
