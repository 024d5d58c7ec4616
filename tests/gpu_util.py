"""Helpers for the GPU parity tests (host-side comparison only)."""

import numpy as np
import pytest
import torch

import oracle

# max |gpu - oracle| / max |oracle| per output tensor, for bf16 compute with
# float32 accumulation against the float64 oracle
TOL = 2e-2


def device():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    return torch.device("cuda:0")


def host_f32(t):
    """bf16/fp32 device tensor -> float32 numpy (exact)."""
    return t.detach().float().cpu().numpy()


def store_np(st):
    torch.cuda.synchronize()
    return (st.codes.cpu().numpy(), st.absmax_q.cpu().numpy(), st.absmax_s2.cpu().numpy())


def oracle_store(w_bf16):
    """Quantize with the oracle from an exact host copy of the bf16 weights."""
    return oracle.quantize(host_f32(w_bf16).ravel())


def assert_store_equal(st, ref, label=""):
    codes, q8, s2 = store_np(st)
    n = ref["numel"]
    assert codes.shape == ref["codes"].shape, label
    bad = np.nonzero(codes != ref["codes"])[0]
    assert bad.size == 0, f"{label}: {bad.size} code bytes differ, first at byte {bad[:5]}"
    assert np.array_equal(q8, ref["absmax_q"]), f"{label}: absmax_q differs"
    assert np.array_equal(s2.view(np.uint32), ref["absmax_s2"].view(np.uint32)), f"{label}: s2 differs"
    assert n == st.numel


def rel_err(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    denom = np.max(np.abs(want))
    if denom == 0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - want)) / denom)


def assert_close(got, want, label, tol=TOL):
    e = rel_err(got, want)
    print(f"[parity] {label}: max rel err {e:.3e} (tol {tol})", flush=True)
    assert e <= tol, f"{label}: max rel err {e:.3e} > {tol}"
    return e


def oracle_wprime(w_bf16):
    ref = oracle_store(w_bf16)
    N, K = w_bf16.shape
    wp = oracle.dequantize(ref["codes"], ref["absmax_q"], ref["absmax_s2"], N * K).reshape(N, K)
    return ref, wp
