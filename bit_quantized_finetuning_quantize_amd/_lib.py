"""Loads libqlora.so (the in-tree HIP build) and declares its C ABI.

The library is required: there is no fallback. Import fails loudly when the
shared object is missing; build it with
`python bit_quantized_finetuning_quantize_amd/build.py`.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqlora.so")

_c_i64 = ctypes.c_int64
_c_i32 = ctypes.c_int32
_c_int = ctypes.c_int
_c_f32 = ctypes.c_float
_c_size = ctypes.c_size_t
_vp = ctypes.c_void_p

# name -> (restype, argtypes); mirrors include/qlora.h
SIGNATURES = {
    "qlora_nf4_codes_bytes": (_c_i64, [_c_i64]),
    "qlora_nf4_num_blocks": (_c_i64, [_c_i64]),
    "qlora_nf4_num_groups": (_c_i64, [_c_i64]),
    "qlora_nf4_codebook": (None, [_vp]),
    "qlora_nf4_quantize": (_c_int, [_vp, _c_i64, _vp, _vp, _vp, _vp]),
    "qlora_nf4_dequantize": (_c_int, [_vp, _vp, _vp, _c_i64, _vp, _vp]),
    "qlora_nf4_dequantize_bf16": (_c_int, [_vp, _vp, _vp, _c_i64, _vp, _vp]),
    "qlora_nf4_quantize_ex": (_c_int, [_vp, _c_i64, _vp, _vp, _vp, _c_i32, _vp]),
    "qlora_nf4_dequantize_ex": (_c_int, [_vp, _vp, _vp, _c_i64, _c_i32, _vp, _vp]),
    "qlora_nf4_dequantize_bf16_ex": (_c_int, [_vp, _vp, _vp, _c_i64, _c_i32, _vp, _vp]),
    "qlora_nf4_merge_ex": (_c_int, [_vp, _vp, _vp, _c_i64, _c_i64, _vp, _vp, _c_i32, _c_f32,
                                    _c_i32, _vp, _vp]),
    "qlora_linear_fwd_ex": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64,
                                     _c_i32, _c_f32, _vp, _vp, _vp, _c_size, _c_i32, _vp]),
    "qlora_linear_bwd_ex": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_i64,
                                     _c_i64, _c_i32, _c_f32, _vp, _vp, _vp, _vp, _c_size,
                                     _c_i32, _vp]),
    "qlora_adamw_step": (_c_int, [_vp, _vp, _vp, _vp, _c_i64, _c_f32, _c_f32, _c_f32, _c_f32,
                                  _c_f32, _c_i64, _vp, _vp]),
    "qlora_adamw8_step": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_f32, _c_f32, _c_f32,
                                   _c_f32, _c_f32, _c_i64, _vp, _vp]),
    "qlora_nf4_merge": (_c_int, [_vp, _vp, _vp, _c_i64, _c_i64, _vp, _vp, _c_i32, _c_f32, _vp,
                                 _vp]),
    "qlora_linear_workspace_bytes": (_c_size, [_c_i64, _c_i64, _c_i64, _c_i32]),
    "qlora_dropout_mask": (_c_int, [_c_i64, _c_i64, _c_f32, ctypes.c_uint64, ctypes.c_uint64, _vp,
                                    _vp]),
    "qlora_linear_fwd_dropout": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64,
                                          _c_i32, _c_f32, _vp, _c_f32, _vp, _vp, _vp, _c_size,
                                          _vp]),
    "qlora_linear_bwd_dropout": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_i64,
                                          _c_i64, _c_i32, _c_f32, _vp, _c_f32, _vp, _vp, _vp, _vp,
                                          _c_size, _vp]),
    "qlora_linear_fwd": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64, _c_i32,
                                  _c_f32, _vp, _vp, _vp, _c_size, _vp]),
    "qlora_linear_bwd": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64,
                                  _c_i32, _c_f32, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "qlora_linear_fwd_noalloc": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64,
                                          _c_i32, _c_f32, _vp, _vp, _vp]),
    "qlora_linear_fwd_profiled": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_i64, _c_i64,
                                           _c_i32, _c_f32, _vp, _vp, _vp, _c_size, _vp, _vp,
                                           _vp]),
    "qlora_linear_bwd_profiled": (_c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i64, _c_i64,
                                           _c_i64, _c_i32, _c_f32, _vp, _vp, _vp, _vp, _c_size,
                                           _vp, _vp, _vp]),
    "qlora_gemv_wait_limit": (_c_int, [_c_i64]),
    "qlora_status_string": (ctypes.c_char_p, [_c_int]),
    "qlora_last_hip_error": (_c_int, []),
}


def load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python bit_quantized_finetuning_quantize_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = load()
