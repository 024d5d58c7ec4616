"""The C-ABI library loads, exports every symbol the header declares, and
rejects bad arguments before touching the GPU (CPU only: no compute calls).

Argument validation in libqlora.so runs before any HIP call, so the
rejected calls below are safe without a device.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlora.h")


@pytest.fixture(scope="module")
def lib():
    from bit_quantized_finetuning_quantize_amd._lib import LIB
    return LIB


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(qlora_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ("qlora_nf4_quantize", "qlora_nf4_dequantize", "qlora_linear_fwd",
              "qlora_linear_bwd"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    from bit_quantized_finetuning_quantize_amd._lib import SIGNATURES
    names = _declared_functions()
    for n in names:
        assert hasattr(lib, n), n
        assert n in SIGNATURES, n


def test_codebook_matches_oracle_bitwise(lib):
    buf = (ctypes.c_float * 16)()
    lib.qlora_nf4_codebook(ctypes.cast(buf, ctypes.c_void_p))
    got = np.frombuffer(buf, dtype=np.float32).copy()
    assert np.array_equal(got.view(np.uint32), oracle.codebook().view(np.uint32))


@pytest.mark.parametrize("numel", [1, 2, 63, 64, 65, 16384, 16385, 4096 * 4096, 22016 * 8192])
def test_store_sizes(lib, numel):
    assert lib.qlora_nf4_codes_bytes(numel) == oracle.codes_bytes(numel)
    assert lib.qlora_nf4_num_blocks(numel) == oracle.num_blocks(numel)
    assert lib.qlora_nf4_num_groups(numel) == oracle.num_groups(numel)
    assert lib.qlora_nf4_codes_bytes(-1) == -1


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4, 7):
        assert isinstance(lib.qlora_status_string(s), bytes)


def test_gemv_wait_limit_range(lib):
    assert lib.qlora_gemv_wait_limit(-1) == -1
    assert lib.qlora_gemv_wait_limit(1000001) == -1
    assert lib.qlora_gemv_wait_limit(0) == 0
    assert lib.qlora_gemv_wait_limit(1000000) == 0
    assert lib.qlora_gemv_wait_limit(200) == 0  # the default, restored


FAKE = ctypes.c_void_p(1 << 20)       # aligned, never dereferenced
ODD = ctypes.c_void_p((1 << 20) + 1)  # misaligned


def test_quantize_rejects(lib):
    q = lib.qlora_nf4_quantize
    assert q(None, 64, FAKE, FAKE, FAKE, None) == -1
    assert q(FAKE, 0, FAKE, FAKE, FAKE, None) == -1
    assert q(FAKE, 64, None, FAKE, FAKE, None) == -1
    assert q(FAKE, 64, FAKE, FAKE, None, None) == -1   # absmax_s2 is always needed
    assert q(FAKE, 64, FAKE, None, None, None) == -1
    assert q(ODD, 64, FAKE, FAKE, FAKE, None) == -2
    assert q(FAKE, 64, ODD, FAKE, FAKE, None) == -2


def test_dequantize_rejects(lib):
    for f in (lib.qlora_nf4_dequantize, lib.qlora_nf4_dequantize_bf16):
        assert f(None, FAKE, FAKE, 64, FAKE, None) == -1
        assert f(FAKE, FAKE, FAKE, -5, FAKE, None) == -1
        assert f(FAKE, FAKE, FAKE, 64, ODD, None) == -2


def _fwd(lib, M=32, N=128, K=128, r=8, ws=FAKE, wsb=1 << 30, X=FAKE, codes=FAKE, A=FAKE):
    return lib.qlora_linear_fwd(X, codes, FAKE, FAKE, A, FAKE, M, N, K, r, 1.0, FAKE, None,
                                ws, wsb, None)


def test_linear_fwd_rejects(lib):
    assert _fwd(lib, X=None) == -1
    assert _fwd(lib, codes=None) == -1
    assert _fwd(lib, M=0) == -1
    assert _fwd(lib, K=100) == -2          # K % 64
    assert _fwd(lib, N=100) == -2          # N % 64
    assert _fwd(lib, r=0) == -2
    assert _fwd(lib, r=257) == -2
    assert _fwd(lib, X=ODD) == -2
    assert _fwd(lib, ws=None) == -3
    assert _fwd(lib, wsb=16) == -3
    # 32-bit operand offsets inside the kernels
    assert _fwd(lib, M=1 << 20, N=1024, K=64) == -2        # M N = 2^30
    assert _fwd(lib, M=1 << 20, N=64, K=1024) == -2        # M K = 2^30
    assert _fwd(lib, M=1, N=(1 << 21) + 64, K=64) == -2    # N above 2^21
    assert _fwd(lib, M=1, N=1 << 21, K=1 << 11) == -2      # N K = 2^32
    assert lib.qlora_linear_workspace_bytes(1, 1 << 21, 1 << 11, 8) == 0


NOALLOC_SCRATCH_BYTES = 32 << 20  # QLORA_NOALLOC_SCRATCH_BYTES in include/qlora.h


def _fwd_noalloc(lib, M=32, N=128, K=128, r=8, X=FAKE, codes=FAKE, A=FAKE):
    return lib.qlora_linear_fwd_noalloc(X, codes, FAKE, FAKE, A, FAKE, M, N, K, r, 1.0, FAKE,
                                        None, None)


def test_header_states_noalloc_scratch_size():
    text = open(HEADER).read()
    m = re.search(r"#define QLORA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == NOALLOC_SCRATCH_BYTES


def test_linear_fwd_noalloc_rejects(lib):
    """The forward without a workspace validates like the forward and rejects
    shapes whose workspace exceeds the fixed scratch array, before any GPU
    call."""
    assert _fwd_noalloc(lib, X=None) == -1
    assert _fwd_noalloc(lib, codes=None) == -1
    assert _fwd_noalloc(lib, M=0) == -1
    assert _fwd_noalloc(lib, K=100) == -2
    assert _fwd_noalloc(lib, r=257) == -2
    assert _fwd_noalloc(lib, X=ODD) == -2
    M, N, K, r = 16384, 22016, 8192, 256
    assert lib.qlora_linear_workspace_bytes(M, N, K, r) > NOALLOC_SCRATCH_BYTES
    assert _fwd_noalloc(lib, M, N, K, r) == -3
    # every workload shape fits
    for M, N, K, r in ((16, 4096, 4096, 16), (2048, 11008, 4096, 64), (2048, 4096, 11008, 64),
                       (4096, 22016, 8192, 64), (4096, 8192, 22016, 64)):
        assert 0 < lib.qlora_linear_workspace_bytes(M, N, K, r) <= NOALLOC_SCRATCH_BYTES


def test_store_type_rejected_outside_range(lib):
    """Every _ex entry point rejects a store type outside [0, 3] before any
    GPU call."""
    for t in (-1, 4, 1 << 20):
        assert lib.qlora_nf4_quantize_ex(FAKE, 64, FAKE, FAKE, FAKE, t, None) == -1
        assert lib.qlora_nf4_dequantize_ex(FAKE, FAKE, FAKE, 64, t, FAKE, None) == -1
        assert lib.qlora_nf4_dequantize_bf16_ex(FAKE, FAKE, FAKE, 64, t, FAKE, None) == -1
        assert lib.qlora_nf4_merge_ex(FAKE, FAKE, FAKE, 64, 64, FAKE, FAKE, 8, 1.0, t, FAKE,
                                      None) == -1
        assert lib.qlora_linear_fwd_ex(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 32, 128, 128, 8, 1.0,
                                       FAKE, None, FAKE, 1 << 30, t, None) == -1
        assert lib.qlora_linear_bwd_ex(FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 32, 128,
                                       128, 8, 1.0, FAKE, FAKE, FAKE, FAKE, 1 << 30, t,
                                       None) == -1
    # a valid type passes validation up to the first shape check
    assert lib.qlora_linear_fwd_ex(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 32, 128, 100, 8, 1.0,
                                   FAKE, None, FAKE, 1 << 30, 3, None) == -2


def test_header_store_type_values():
    text = open(HEADER).read()
    for name, v in (("QLORA_STORE_NF4", 0), ("QLORA_STORE_FP4", 1), ("QLORA_STORE_DQ_FP8", 2)):
        assert re.search(rf"#define {name} {v}\b", text), name


def test_linear_bwd_rejects(lib):
    b = lib.qlora_linear_bwd
    args = [FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 32, 128, 128, 8, 1.0, FAKE, FAKE,
            FAKE, FAKE, 1 << 30, None]
    bad = list(args); bad[14] = None  # dA
    assert b(*bad) == -1
    bad = list(args); bad[10] = 96    # K % 64
    assert b(*bad) == -2
    bad = list(args); bad[17] = 8     # workspace too small
    assert b(*bad) == -3


def test_workspace_query(lib):
    assert lib.qlora_linear_workspace_bytes(16, 4096, 4096, 16) > 0
    assert lib.qlora_linear_workspace_bytes(2048, 11008, 4096, 64) > 0
    assert lib.qlora_linear_workspace_bytes(16, 4096, 4000, 16) == 0


def _merge(lib, N=128, K=128, r=8, codes=FAKE, A=FAKE, out=FAKE, s2=FAKE):
    return lib.qlora_nf4_merge(codes, FAKE, s2, N, K, A, FAKE, r, 0.25, out, None)


def test_workspace_serves_smaller_linears(lib):
    """A workspace sized for a linear serves every linear of the same token
    count and rank with no larger K and N (the split-K partial buffer is
    sized by a bound that grows with K and N), so one workspace sized for a
    model's largest linear serves all of them."""
    dims = [64, 192, 256, 1024, 4096, 8192, 11008, 22016]
    for M in (17, 300, 2048, 4096):
        for r in (8, 64, 100):
            size = {(N, K): lib.qlora_linear_workspace_bytes(M, N, K, r)
                    for N in dims for K in dims}
            for (N, K), b in size.items():
                for (N2, K2), b2 in size.items():
                    if N <= N2 and K <= K2:
                        assert b <= b2, (M, r, N, K, N2, K2, b, b2)


def test_merge_rejects(lib):
    assert _merge(lib, codes=None) == -1
    assert _merge(lib, A=None) == -1
    assert _merge(lib, out=None) == -1
    assert _merge(lib, N=0) == -1
    assert _merge(lib, K=-64) == -1
    assert _merge(lib, K=100) == -2        # K % 64
    assert _merge(lib, r=0) == -2
    assert _merge(lib, r=257) == -2
    assert _merge(lib, out=ODD) == -2
    assert _merge(lib, codes=ODD) == -2
    assert _merge(lib, N=65536 * 64 + 1) == -2   # more than 65535 row tiles


def test_adamw_rejects(lib):
    a = lib.qlora_adamw_step
    ok = [FAKE, FAKE, FAKE, FAKE, 16, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, None, None]
    bad = list(ok); bad[0] = None
    assert a(*bad) == -1
    bad = list(ok); bad[4] = 0
    assert a(*bad) == -1
    bad = list(ok); bad[10] = 0      # step counts from 1
    assert a(*bad) == -1
    bad = list(ok); bad[6] = 1.0     # beta1 outside [0, 1)
    assert a(*bad) == -1
    bad = list(ok); bad[8] = 0.0     # eps
    assert a(*bad) == -1
    bad = list(ok); bad[1] = ODD
    assert a(*bad) == -2


def test_dropout_mask_rejects(lib):
    m = lib.qlora_dropout_mask
    assert m(4, 64, 0.05, 1, 0, None, None) == -1          # null mask
    assert m(0, 64, 0.05, 1, 0, FAKE, None) == -1          # M
    assert m(4, 64, -0.1, 1, 0, FAKE, None) == -1          # p < 0
    assert m(4, 64, 1.0, 1, 0, FAKE, None) == -1           # p = 1
    assert m(4, 64, float("nan"), 1, 0, FAKE, None) == -1
    assert m(4, 48, 0.05, 1, 0, FAKE, None) == -2          # K % 32
    assert m(4, 64, 0.99999994, 1, 0, FAKE, None) == -2    # rounds to certain dropping
    assert m(4, 64, 0.05, 1, 0, ODD, None) == -2           # alignment


def test_linear_dropout_rejects(lib):
    f = lib.qlora_linear_fwd_dropout
    fa = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 32, 128, 128, 8, 1.0, FAKE, 0.05, FAKE, None, FAKE,
          1 << 30, None]
    bad = list(fa); bad[11] = None     # keep mask
    assert f(*bad) == -1
    bad = list(fa); bad[12] = 1.5      # p
    assert f(*bad) == -1
    bad = list(fa); bad[11] = ODD
    assert f(*bad) == -2
    bad = list(fa); bad[8] = 96        # K % 64
    assert f(*bad) == -2
    bad = list(fa); bad[16] = 8        # workspace
    assert f(*bad) == -3
    b = lib.qlora_linear_bwd_dropout
    ba = [FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 32, 128, 128, 8, 1.0, FAKE, 0.05, FAKE,
          FAKE, FAKE, FAKE, 1 << 30, None]
    bad = list(ba); bad[13] = None
    assert b(*bad) == -1
    bad = list(ba); bad[11] = 256      # masked input gradient above rank 192
    assert b(*bad) == -2
    bad = list(ba); bad[14] = -0.5
    assert b(*bad) == -1
    bad = list(ba); bad[19] = 8
    assert b(*bad) == -3


def test_adamw8_rejects(lib):
    a = lib.qlora_adamw8_step
    ok = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 300, 1e-3, 0.9, 0.999, 1e-8, 0.0, 1, None, None]
    bad = list(ok); bad[1] = None      # m8
    assert a(*bad) == -1
    bad = list(ok); bad[4] = None      # v_scale
    assert a(*bad) == -1
    bad = list(ok); bad[6] = 0
    assert a(*bad) == -1
    bad = list(ok); bad[12] = 0        # step counts from 1
    assert a(*bad) == -1
    bad = list(ok); bad[9] = 1.0       # beta2 outside [0, 1)
    assert a(*bad) == -1
    bad = list(ok); bad[2] = ODD       # a scale array not 4-byte aligned
    assert a(*bad) == -2
    bad = list(ok); bad[13] = ODD      # bf16 copy not 2-byte aligned
    assert a(*bad) == -2
