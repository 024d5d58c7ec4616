"""bfloat16 rounding for the oracle (TEST INFRASTRUCTURE ONLY).

[P2] "Training Flow" and [P4] "A code example with common libraries" fix the
compute dtype as bfloat16: the dequantized weight is rounded to bfloat16
before the matrix product. bfloat16 is the upper half of an IEEE binary32;
rounding to it is round-to-nearest, ties-to-even on the 16 dropped bits.

Pinned by tests against torch's own float32 -> bfloat16 conversion on
exhaustive bit patterns near every tie, and on random values.
"""

import numpy as np


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (RNE); return the 16-bit patterns."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    lower = u & 0xFFFF
    upper = u >> 16
    # round half to even on the dropped half-word
    round_up = (lower > 0x8000) | ((lower == 0x8000) & ((upper & 1) == 1))
    out = upper + round_up.astype(np.uint64)
    nan = np.isnan(x)
    out = np.where(nan, (upper | 0x40), out)  # keep a quiet NaN
    return out.astype(np.uint16)


def bf16_bits_to_f32(b):
    """Widen bfloat16 bit patterns to the float32 values they denote (exact)."""
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_round(x):
    """float32 -> nearest bfloat16 value (RNE), returned as float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x)).reshape(np.shape(x))
