"""Stored 4-bit tensors of every type the library handles (TEST
INFRASTRUCTURE ONLY): the level table (NF4 or FP4) crossed with the code of
the block constants (an 8-bit linear code, an 8-bit floating-point code, or
none).

Store types (bit flags, as the library's QLORA_STORE_* values):
  0  NF4 levels, 8-bit linear constant code (oracle.nf4.quantize)
  1  FP4 levels (oracle.fp4) instead of NF4
  2  8-bit floating-point constant code instead of the linear one
Without double quantization (absmax_q = None) the constant code does not
apply: each block keeps its float32 constant.

Level 1 is the same for every type ([P4] "Step 1", "Step 2"): blocks of 64
consecutive values, c = max |w|, n = fl32(w / c), each value replaced by the
code of the nearest level (NF4: oracle.nf4.nearest_level; FP4:
oracle.fp4.nearest_code); an all-zero block takes the code of level 0.

Level 2 ([P4] "Step 3": the block constants quantized again to 8 bits in
groups of 256, each group with one float32 second-level constant; the pages
do not say which 8-bit code). Two readings:
  linear  s2 = max c; q8 = round_half_even(255 fl32(c / s2));
          c' = fl32(fl32(q8 / 255) s2)                     (oracle.nf4)
  fp8     the OCP E4M3 code (oracle.fp8) of the constant relative to a
          per-group scale, as the optimizer's 8-bit state is stored:
          S = fl32(max c / 448); q8 = E4M3(fl32(c / S)) (nearest, ties to
          even, saturating at 448); c' = fl32(dec(q8) S); S = 0 gives q8 = 0.
          absmax_s2 holds S. Four mantissa bits' worth of relative precision
          down to 2^-6 of the group maximum, where the linear code loses it
          (|c - c'| <= s2 / 510 is a large relative error for small c).

Dequantized value ([P4] "A worked example" step 4, "Step 5"):
  w' = fl32(L[q] c')
with L the level table in code order.

Pinned by: type 0 equal to oracle.nf4.quantize / dequantize; the FP4 and
E4M3 pieces by their own modules' pins (oracle.fp4, oracle.fp8 against
torch's float8 conversions); the fp8 second level by the group maximum
decoding to (about) 448 S, the relative half-step bound and the zero group.
"""

import numpy as np

from . import fp4 as _fp4
from . import fp8 as _fp8
from .nf4 import BLOCK, GROUP, codebook as nf4_codebook, nearest_level, pack_codes, \
    unpack_codes, _block_absmax, level8

FP4 = 1
DQ_FP8 = 2
E4M3_TOP = 448.0


def levels(store_type):
    """The 16 levels in code order."""
    return _fp4.codebook() if store_type & FP4 else nf4_codebook()


def zero_code(store_type):
    return _fp4.ZERO_CODE if store_type & FP4 else int(nearest_level(np.float32(0.0)))


def _codes(w, absmax, store_type, chunk=1 << 20):
    numel = w.size
    q = np.empty(numel, dtype=np.uint8)
    lv = levels(store_type)
    z = zero_code(store_type)
    for s in range(0, numel, chunk):
        e = min(numel, s + chunk)
        c = absmax[np.arange(s, e) // BLOCK]
        safe = np.where(c == 0, np.float32(1.0), c).astype(np.float32)
        n = (w[s:e] / safe).astype(np.float32)  # one IEEE float32 division
        qq = _fp4.nearest_code(n, lv) if store_type & FP4 else nearest_level(n, lv)
        qq[c == 0] = z
        q[s:e] = qq
    return q


def _second_level(absmax, store_type):
    nb = absmax.size
    ng = -(-nb // GROUP)
    padded = np.zeros(ng * GROUP, dtype=np.float32)
    padded[:nb] = absmax
    gmax = padded.reshape(ng, GROUP).max(axis=1).astype(np.float32)
    g = np.arange(nb) // GROUP
    if store_type & DQ_FP8:
        S = (gmax / np.float32(E4M3_TOP)).astype(np.float32)       # fl32(max / 448)
        safe = np.where(S[g] == 0, np.float32(1.0), S[g]).astype(np.float32)
        r = (absmax / safe).astype(np.float32)                     # fl32(c / S)
        q8 = _fp8.encode(r, _fp8.E4M3)
        q8[S[g] == 0] = 0
        return q8, S
    denom = np.where(gmax[g] == 0, np.float32(1.0), gmax[g]).astype(np.float32)
    ratio = (absmax / denom).astype(np.float32)
    scaled = (ratio * np.float32(255.0)).astype(np.float32)
    q8 = np.clip(np.rint(scaled), 0, 255).astype(np.uint8)
    q8[gmax[g] == 0] = 0
    return q8, gmax


def quantize(w, store_type=0, double_quant=True):
    """Quantize a flat float32 array (bf16-exact values). Returns codes,
    absmax_q (None without double quantization), absmax_s2 and the
    unpacked codes q."""
    w = np.ascontiguousarray(np.asarray(w, dtype=np.float32).ravel())
    absmax = _block_absmax(w)
    q = _codes(w, absmax, store_type)
    if not double_quant:
        return {"codes": pack_codes(q), "absmax_q": None, "absmax_s2": absmax.copy(),
                "absmax": absmax, "q": q, "numel": w.size}
    q8, s2 = _second_level(absmax, store_type)
    return {"codes": pack_codes(q), "absmax_q": q8, "absmax_s2": s2, "absmax": absmax,
            "q": q, "numel": w.size}


def block_constants(absmax_q, absmax_s2, store_type=0):
    """c' per block."""
    s2 = np.asarray(absmax_s2, dtype=np.float32)
    if absmax_q is None:
        return s2
    q8 = np.asarray(absmax_q, dtype=np.uint8)
    g = np.arange(q8.size) // GROUP
    if store_type & DQ_FP8:
        return (_fp8.decode(q8, _fp8.E4M3) * s2[g]).astype(np.float32)  # dec exact
    return (level8()[q8] * s2[g]).astype(np.float32)


def dequantize(codes, absmax_q, absmax_s2, numel, store_type=0):
    """float32 w' = fl32(L[q] c')."""
    lv = levels(store_type)
    q = unpack_codes(codes, numel)
    cp = block_constants(absmax_q, absmax_s2, store_type)
    return (lv[q] * cp[np.arange(numel) // BLOCK]).astype(np.float32)
