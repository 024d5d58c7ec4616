"""LoRA dropout on the adapter input: the keep mask and its scale.

TEST INFRASTRUCTURE ONLY.

The pages' training recipe sets a LoRA dropout of 0.05 ([P4] "A code example
with common libraries", its LoraConfig; "Practical guidance and best
practices", Adapter settings: a small dropout rate when data is scarce).
Reading taken here: inverted dropout on the input of the adapter path only,
the frozen-weight product sees X unchanged:

    D(X) = (X o keep) * keep_scale,      Y = X W'^T + s D(X) A B

where keep is a 0/1 mask drawn independently per element and keep_scale is
the inverse of the keep probability, so that E[D(X)] = X.

Random numbers: Philox4x32-10 (see oracle.philox) with key = the 64-bit seed
(low word first) and counter = (g mod 2^32, g div 2^32, offset mod 2^32,
offset div 2^32) for group g of eight consecutive elements of X in row-major
order (element e = m K + k belongs to group e div 8). The generator's four
output words give eight 16-bit values, word w holding elements 8g + 2w (low
half) and 8g + 2w + 1 (high half). An element is kept when its value is at
least thr = floor(p 2^16 + 1/2), so the drop probability realized is exactly
thr / 2^16 (0.0500030518 for p = 0.05), and keep_scale = 2^16 / (2^16 - thr).

Packed form: uint32 [M, K/32], bit j of word w of row m is keep[m, 32 w + j].

Pinned by: the generator's known-answer vectors (oracle.philox); p = 0 keeps
everything; the dropped fraction for p = 0.05 on four million elements lies
within six binomial standard deviations of thr / 2^16; masks of different
seeds or offsets differ; the mask of an [M, K] input is the leading rows of
the mask of any taller input with the same K.
"""

import numpy as np

from .philox import philox4x32_10

GROUP_ELEMS = 8


def keep_threshold(p):
    """16-bit threshold of a drop probability p (float32 argument)."""
    p = float(np.float32(p))
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must lie in [0, 1)")
    thr = int(np.floor(p * 65536.0 + 0.5))
    if thr >= 65536:
        raise ValueError("dropout probability rounds to 1")
    return thr


def keep_scale(p):
    """Exact inverse of the realized keep probability (float64)."""
    thr = keep_threshold(p)
    return 65536.0 / (65536 - thr)


def dropout_keep(M, K, p, seed, offset=0):
    """bool [M, K]: True where element (m, k) of the adapter input is kept."""
    n = M * K
    if n % GROUP_ELEMS:
        raise ValueError("M K must be a multiple of 8")
    thr = keep_threshold(p)
    g = np.arange(n // GROUP_ELEMS, dtype=np.uint64)
    ctr = np.empty(g.shape + (4,), dtype=np.uint32)
    ctr[:, 0] = (g & np.uint64(0xFFFFFFFF)).astype(np.uint32)
    ctr[:, 1] = (g >> np.uint64(32)).astype(np.uint32)
    ctr[:, 2] = offset & 0xFFFFFFFF
    ctr[:, 3] = (offset >> 32) & 0xFFFFFFFF
    x = philox4x32_10(ctr, (seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF))
    halves = np.empty((g.size, 8), dtype=np.uint32)
    halves[:, 0::2] = x & 0xFFFF
    halves[:, 1::2] = x >> 16
    return (halves >= thr).reshape(M, K)


def pack_keep(keep):
    """bool [M, K] -> uint32 [M, K/32] (bit j of word w = keep[m, 32 w + j])."""
    keep = np.asarray(keep, dtype=bool)
    M, K = keep.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    bits = keep.reshape(M, K // 32, 32).astype(np.uint64)
    weights = np.uint64(1) << np.arange(32, dtype=np.uint64)
    return (bits * weights).sum(axis=-1).astype(np.uint32)


def unpack_keep(words, K):
    words = np.asarray(words, dtype=np.uint32)
    M = words.shape[0]
    j = np.arange(32, dtype=np.uint32)
    bits = (words[:, :, None] >> j) & np.uint32(1)
    return bits.reshape(M, -1)[:, :K].astype(bool)
