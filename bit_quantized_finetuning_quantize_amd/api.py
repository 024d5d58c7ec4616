"""Thin Python binding over the C ABI (argument marshalling only).

Every computation runs in libqlora.so on the caller's current HIP stream;
torch is used only to hold device memory and to name the stream. Function
names match include/qlora.h.
"""

import ctypes

import torch

from ._lib import LIB

BLOCK = 64
GROUP = 256
# store types (include/qlora.h): bit flags
STORE_NF4 = 0
STORE_FP4 = 1
STORE_DQ_FP8 = 2


class QloraError(RuntimeError):
    pass


def _check(status):
    if status != 0:
        msg = LIB.qlora_status_string(status).decode()
        hip = LIB.qlora_last_hip_error() if status == -4 else 0
        raise QloraError(f"qlora status {status}: {msg}" + (f" (hipError {hip})" if hip else ""))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


_HIP = None


def _state_ptr(t, name):
    """Device-side address of an optimizer-state tensor: a contiguous GPU
    tensor, or a contiguous pinned host tensor (hipHostMalloc, e.g. torch's
    pin_memory=True), which the kernel then reads and writes over the host
    link; its device address comes from hipHostGetDevicePointer."""
    global _HIP
    if not t.is_contiguous():
        raise QloraError(f"{name} must be contiguous")
    if t.is_cuda:
        return ctypes.c_void_p(t.data_ptr())
    if not t.is_pinned():
        raise QloraError(f"{name} on the host must be pinned memory (pin_memory=True)")
    if _HIP is None:
        _HIP = ctypes.CDLL("libamdhip64.so")
        _HIP.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p,
                                                 ctypes.c_uint]
        _HIP.hipHostGetDevicePointer.restype = ctypes.c_int
    dptr = ctypes.c_void_p()
    rc = _HIP.hipHostGetDevicePointer(ctypes.byref(dptr), ctypes.c_void_p(t.data_ptr()), 0)
    if rc != 0 or not dptr.value:
        raise QloraError(f"{name}: hipHostGetDevicePointer failed ({rc})")
    return dptr


def _need(t, dtype, name):
    if t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise QloraError(f"{name} must be a contiguous {dtype} tensor on the GPU")


def qlora_nf4_codes_bytes(numel):
    return int(LIB.qlora_nf4_codes_bytes(numel))


def qlora_nf4_num_blocks(numel):
    return int(LIB.qlora_nf4_num_blocks(numel))


def qlora_nf4_num_groups(numel):
    return int(LIB.qlora_nf4_num_groups(numel))


def qlora_nf4_codebook():
    buf = (ctypes.c_float * 16)()
    LIB.qlora_nf4_codebook(ctypes.cast(buf, ctypes.c_void_p))
    return list(buf)


class Nf4Store:
    """The device buffers of one 4-bit tensor (owned by torch). Without
    double quantization `absmax_q` is None and `absmax_s2` holds one float32
    constant per 64-block. `store_type`: STORE_NF4 (0), or the flags
    STORE_FP4 (FP4 levels) and STORE_DQ_FP8 (E4M3 constant code)."""

    def __init__(self, codes, absmax_q, absmax_s2, numel, shape=None, store_type=STORE_NF4):
        self.codes, self.absmax_q, self.absmax_s2 = codes, absmax_q, absmax_s2
        self.numel = int(numel)
        self.shape = tuple(shape) if shape is not None else (self.numel,)
        self.store_type = int(store_type)

    @property
    def double_quant(self):
        return self.absmax_q is not None

    def nbytes(self):
        q8 = self.absmax_q.numel() if self.absmax_q is not None else 0
        return self.codes.numel() + q8 + 4 * self.absmax_s2.numel()


def empty_store(numel, device, shape=None, double_quant=True, store_type=STORE_NF4):
    codes = torch.empty(qlora_nf4_codes_bytes(numel), dtype=torch.uint8, device=device)
    if double_quant:
        q8 = torch.empty(qlora_nf4_num_blocks(numel), dtype=torch.uint8, device=device)
        s2 = torch.empty(qlora_nf4_num_groups(numel), dtype=torch.float32, device=device)
    else:
        q8 = None
        s2 = torch.empty(qlora_nf4_num_blocks(numel), dtype=torch.float32, device=device)
    return Nf4Store(codes, q8, s2, numel, shape, store_type)


def qlora_nf4_quantize(w, out=None, double_quant=True, store_type=STORE_NF4):
    """Quantize a bf16 tensor (any shape, flattened row-major); with
    double_quant=False the store keeps the float32 block constants;
    store_type selects FP4 levels and / or the E4M3 constant code."""
    _need(w, torch.bfloat16, "w")
    if out is None:
        st = empty_store(w.numel(), w.device, w.shape, double_quant, store_type)
    else:
        st = out
        st.store_type = int(store_type)
    _check(LIB.qlora_nf4_quantize_ex(_ptr(w), w.numel(), _ptr(st.codes), _ptr(st.absmax_q),
                                     _ptr(st.absmax_s2), st.store_type, _stream()))
    return st


def qlora_nf4_dequantize(st, out=None):
    out = out if out is not None else torch.empty(st.numel, dtype=torch.float32,
                                                  device=st.codes.device)
    _check(LIB.qlora_nf4_dequantize_ex(_ptr(st.codes), _ptr(st.absmax_q), _ptr(st.absmax_s2),
                                       st.numel, st.store_type, _ptr(out), _stream()))
    return out


def qlora_nf4_dequantize_bf16(st, out=None):
    out = out if out is not None else torch.empty(st.numel, dtype=torch.bfloat16,
                                                  device=st.codes.device)
    _check(LIB.qlora_nf4_dequantize_bf16_ex(_ptr(st.codes), _ptr(st.absmax_q),
                                            _ptr(st.absmax_s2), st.numel, st.store_type,
                                            _ptr(out), _stream()))
    return out


def qlora_nf4_merge(st, A, B, scale, out=None):
    """bf16(w' + scale (A B)^T) for a store of W [N x K]: the adapter folded
    into a 16-bit copy of the frozen weight; returns bf16 [N x K]."""
    N, K = st.shape
    r = A.shape[1]
    out = out if out is not None else torch.empty(N, K, dtype=torch.bfloat16,
                                                  device=st.codes.device)
    _check(LIB.qlora_nf4_merge_ex(_ptr(st.codes), _ptr(st.absmax_q), _ptr(st.absmax_s2), N, K,
                                  _ptr(A), _ptr(B), r, float(scale), st.store_type, _ptr(out),
                                  _stream()))
    return out


def qlora_adamw_step(p, m, v, g, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0,
                     step=1, p_bf16=None):
    """One AdamW step in place on float32 p, m, v with gradient g (same
    number of elements); writes bf16(p) into p_bf16 when given."""
    n = p.numel()
    for t in (m, v, g):
        if t.numel() != n or t.dtype != torch.float32:
            raise QloraError("p, m, v, g must be float32 tensors of one size")
    if p_bf16 is not None and p_bf16.numel() != n:
        raise QloraError("p_bf16 must have as many elements as p")
    _check(LIB.qlora_adamw_step(_ptr(p), _state_ptr(m, "m"), _state_ptr(v, "v"), _ptr(g), n,
                                float(lr), float(beta1),
                                float(beta2), float(eps), float(weight_decay), int(step),
                                _ptr(p_bf16) if p_bf16 is not None else None, _stream()))


def adamw_state(n, device, host=False):
    """Zero float32 AdamW moments (m, v) for n parameters, on the GPU or
    (host=True) in pinned host memory."""
    if host:
        return tuple(torch.zeros(n, dtype=torch.float32, pin_memory=True) for _ in range(2))
    return tuple(torch.zeros(n, dtype=torch.float32, device=device) for _ in range(2))


def adamw8_state(n, device, host=False):
    """Zero 8-bit AdamW state for n parameters: (m8, m_scale, v8, v_scale),
    on the GPU or (host=True) in pinned host memory."""
    nb = (n + 255) // 256
    kw = dict(pin_memory=True) if host else dict(device=device)
    return (torch.zeros(n, dtype=torch.uint8, **kw),
            torch.zeros(nb, dtype=torch.float32, **kw),
            torch.zeros(n, dtype=torch.uint8, **kw),
            torch.zeros(nb, dtype=torch.float32, **kw))


def qlora_adamw8_step(p, m8, m_scale, v8, v_scale, g, lr, beta1=0.9, beta2=0.999, eps=1e-8,
                      weight_decay=0.0, step=1, p_bf16=None):
    """One AdamW step with 8-bit moments (all tensors updated in place)."""
    n = p.numel()
    _need(p, torch.float32, "p")
    _need(g, torch.float32, "g")
    for t, dt, name in ((m_scale, torch.float32, "m_scale"), (v_scale, torch.float32, "v_scale"),
                        (m8, torch.uint8, "m8"), (v8, torch.uint8, "v8")):
        if t.dtype != dt:
            raise QloraError(f"{name} must be a {dt} tensor")
    if g.numel() != n or m8.numel() != n or v8.numel() != n:
        raise QloraError("p, g, m8 and v8 must have the same number of elements")
    if m_scale.numel() != (n + 255) // 256 or v_scale.numel() != (n + 255) // 256:
        raise QloraError("one scale per block of 256 parameters")
    if p_bf16 is not None:
        _need(p_bf16, torch.bfloat16, "p_bf16")
    _check(LIB.qlora_adamw8_step(_ptr(p), _state_ptr(m8, "m8"), _state_ptr(m_scale, "m_scale"),
                                 _state_ptr(v8, "v8"), _state_ptr(v_scale, "v_scale"),
                                 _ptr(g), n, float(lr), float(beta1), float(beta2), float(eps),
                                 float(weight_decay), int(step),
                                 _ptr(p_bf16) if p_bf16 is not None else None, _stream()))


def qlora_linear_workspace_bytes(M, N, K, r):
    return int(LIB.qlora_linear_workspace_bytes(M, N, K, r))


def qlora_gemv_wait_limit(microseconds):
    _check(LIB.qlora_gemv_wait_limit(int(microseconds)))


def workspace(M, N, K, r, device):
    n = qlora_linear_workspace_bytes(M, N, K, r)
    if n == 0:
        raise QloraError(f"unsupported linear shape M={M} N={N} K={K} r={r}")
    return torch.empty(n, dtype=torch.uint8, device=device)


def qlora_linear_fwd(X, W, A, B, scale, want_T=True, Y=None, T=None, ws=None, events=None):
    """Y = X bf16(W')^T + scale (X A) B; returns (Y, T) with T fp32 or None.

    `events`: optional (begin, end) raw hipEvent_t handles recorded around
    the dominant kernel (profiling)."""
    M, K = X.shape
    N = W.shape[0]
    r = A.shape[1]
    for t, name in ((X, "X"), (A, "A"), (B, "B")):
        _need(t, torch.bfloat16, name)
    Y = Y if Y is not None else torch.empty(M, N, dtype=torch.bfloat16, device=X.device)
    if want_T and T is None:
        T = torch.empty(M, r, dtype=torch.float32, device=X.device)
    ws = ws if ws is not None else workspace(M, N, K, r, X.device)
    if W.store_type != STORE_NF4:
        if events is not None:
            raise QloraError("profiling events are taken on NF4 stores only")
        _check(LIB.qlora_linear_fwd_ex(_ptr(X), _ptr(W.codes), _ptr(W.absmax_q),
                                       _ptr(W.absmax_s2), _ptr(A), _ptr(B), M, N, K, r,
                                       float(scale), _ptr(Y), _ptr(T) if want_T else None,
                                       _ptr(ws), ws.numel(), W.store_type, _stream()))
        return Y, (T if want_T else None)
    ev = events if events is not None else (None, None)
    _check(LIB.qlora_linear_fwd_profiled(_ptr(X), _ptr(W.codes), _ptr(W.absmax_q),
                                         _ptr(W.absmax_s2), _ptr(A), _ptr(B), M, N, K, r,
                                         float(scale), _ptr(Y), _ptr(T) if want_T else None,
                                         _ptr(ws), ws.numel(), _stream(), ev[0], ev[1]))
    return Y, (T if want_T else None)


def qlora_linear_fwd_noalloc(X, W, A, B, scale, want_T=True, Y=None, T=None):
    """qlora_linear_fwd without a workspace: the library's fixed per-device
    scratch array serves as one (calls that overlap on one GPU race)."""
    M, K = X.shape
    N = W.shape[0]
    r = A.shape[1]
    for t, name in ((X, "X"), (A, "A"), (B, "B")):
        _need(t, torch.bfloat16, name)
    Y = Y if Y is not None else torch.empty(M, N, dtype=torch.bfloat16, device=X.device)
    if want_T and T is None:
        T = torch.empty(M, r, dtype=torch.float32, device=X.device)
    _check(LIB.qlora_linear_fwd_noalloc(_ptr(X), _ptr(W.codes), _ptr(W.absmax_q),
                                        _ptr(W.absmax_s2), _ptr(A), _ptr(B), M, N, K, r,
                                        float(scale), _ptr(Y), _ptr(T) if want_T else None,
                                        _stream()))
    return Y, (T if want_T else None)


def qlora_linear_bwd(dY, X, T, W, A, B, scale, want_dX=True, dX=None, dA=None, dB=None, ws=None,
                     events=None):
    """Returns (dX or None, dA fp32 [K x r], dB fp32 [r x N]).

    `events`: optional (begin, end) raw hipEvent_t handles recorded around
    the input-gradient kernel (profiling)."""
    M, N = dY.shape
    K = X.shape[1]
    r = A.shape[1]
    for t, name in ((dY, "dY"), (X, "X"), (A, "A"), (B, "B")):
        _need(t, torch.bfloat16, name)
    if want_dX and dX is None:
        dX = torch.empty(M, K, dtype=torch.bfloat16, device=X.device)
    dA = dA if dA is not None else torch.empty(K, r, dtype=torch.float32, device=X.device)
    dB = dB if dB is not None else torch.empty(r, N, dtype=torch.float32, device=X.device)
    ws = ws if ws is not None else workspace(M, N, K, r, X.device)
    if W.store_type != STORE_NF4:
        if events is not None:
            raise QloraError("profiling events are taken on NF4 stores only")
        _check(LIB.qlora_linear_bwd_ex(_ptr(dY), _ptr(X), _ptr(T), _ptr(W.codes),
                                       _ptr(W.absmax_q), _ptr(W.absmax_s2), _ptr(A), _ptr(B),
                                       M, N, K, r, float(scale), _ptr(dX) if want_dX else None,
                                       _ptr(dA), _ptr(dB), _ptr(ws), ws.numel(), W.store_type,
                                       _stream()))
        return (dX if want_dX else None), dA, dB
    ev = events if events is not None else (None, None)
    _check(LIB.qlora_linear_bwd_profiled(_ptr(dY), _ptr(X), _ptr(T), _ptr(W.codes),
                                         _ptr(W.absmax_q), _ptr(W.absmax_s2), _ptr(A), _ptr(B),
                                         M, N, K, r, float(scale), _ptr(dX) if want_dX else None,
                                         _ptr(dA), _ptr(dB), _ptr(ws), ws.numel(), _stream(),
                                         ev[0], ev[1]))
    return (dX if want_dX else None), dA, dB


def qlora_dropout_mask(M, K, p, seed, offset=0, out=None, device=None):
    """Keep mask of LoRA dropout over an [M x K] adapter input: int32 tensor
    [M, K // 32] holding the uint32 bit words (bit j of word w of row m keeps
    element (m, 32 w + j))."""
    if out is None:
        dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
        out = torch.empty(M, K // 32, dtype=torch.int32, device=dev)
    _need(out, torch.int32, "mask")
    _check(LIB.qlora_dropout_mask(M, K, float(p), int(seed) & (2**64 - 1),
                                  int(offset) & (2**64 - 1), _ptr(out), _stream()))
    return out


def qlora_linear_fwd_dropout(X, W, A, B, scale, keep_mask, p, want_T=True, Y=None, T=None,
                             ws=None):
    """qlora_linear_fwd with LoRA dropout on the adapter input; returns
    (Y, T) with T = D(X) A (fp32) or None."""
    M, K = X.shape
    N = W.shape[0]
    r = A.shape[1]
    for t, name in ((X, "X"), (A, "A"), (B, "B")):
        _need(t, torch.bfloat16, name)
    _need(keep_mask, torch.int32, "keep_mask")
    Y = Y if Y is not None else torch.empty(M, N, dtype=torch.bfloat16, device=X.device)
    if want_T and T is None:
        T = torch.empty(M, r, dtype=torch.float32, device=X.device)
    ws = ws if ws is not None else workspace(M, N, K, r, X.device)
    _check(LIB.qlora_linear_fwd_dropout(_ptr(X), _ptr(W.codes), _ptr(W.absmax_q),
                                        _ptr(W.absmax_s2), _ptr(A), _ptr(B), M, N, K, r,
                                        float(scale), _ptr(keep_mask), float(p), _ptr(Y),
                                        _ptr(T) if want_T else None, _ptr(ws), ws.numel(),
                                        _stream()))
    return Y, (T if want_T else None)


def qlora_linear_bwd_dropout(dY, X, T, W, A, B, scale, keep_mask, p, want_dX=True, dX=None,
                             dA=None, dB=None, ws=None):
    """qlora_linear_bwd with LoRA dropout; returns (dX or None, dA, dB)."""
    M, N = dY.shape
    K = X.shape[1]
    r = A.shape[1]
    for t, name in ((dY, "dY"), (X, "X"), (A, "A"), (B, "B")):
        _need(t, torch.bfloat16, name)
    _need(keep_mask, torch.int32, "keep_mask")
    if want_dX and dX is None:
        dX = torch.empty(M, K, dtype=torch.bfloat16, device=X.device)
    dA = dA if dA is not None else torch.empty(K, r, dtype=torch.float32, device=X.device)
    dB = dB if dB is not None else torch.empty(r, N, dtype=torch.float32, device=X.device)
    ws = ws if ws is not None else workspace(M, N, K, r, X.device)
    _check(LIB.qlora_linear_bwd_dropout(_ptr(dY), _ptr(X), _ptr(T), _ptr(W.codes),
                                        _ptr(W.absmax_q), _ptr(W.absmax_s2), _ptr(A), _ptr(B),
                                        M, N, K, r, float(scale), _ptr(keep_mask), float(p),
                                        _ptr(dX) if want_dX else None, _ptr(dA), _ptr(dB),
                                        _ptr(ws), ws.numel(), _stream()))
    return (dX if want_dX else None), dA, dB
