"""Philox4x32-10 counter-based random numbers.

TEST INFRASTRUCTURE ONLY.

Definition: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel
random numbers: as easy as 1, 2, 3", SC'11, the Philox family with N = 4
words of 32 bits and ten rounds. A round takes the counter words
(c0, c1, c2, c3) and the two key words (k0, k1) to

    (hi(B * c2) ^ c1 ^ k0,  lo(B * c2),  hi(A * c0) ^ c3 ^ k1,  lo(A * c0))

with A = 0xD2511F53 and B = 0xCD9E8D57 (hi/lo: upper and lower 32 bits of
the 64-bit product); between rounds the key is advanced by the Weyl
constants (0x9E3779B9, 0xBB67AE85), modulo 2^32.

The library implements the same definition in its own HIP code; the two share
nothing but the published definition. Pinned by the published known-answer
vectors of the generator (zero counter and key, all-ones counter and key, and
the digits-of-pi case).
"""

import numpy as np

_MUL0 = np.uint64(0xD2511F53)
_MUL1 = np.uint64(0xCD9E8D57)
_WEYL0 = 0x9E3779B9
_WEYL1 = 0xBB67AE85
_LO = np.uint64(0xFFFFFFFF)
_SH = np.uint64(32)


def philox4x32_10(counter, key):
    """counter: uint32 array [..., 4]; key: two 32-bit integers.
    Returns uint32 [..., 4]: the generator's output for each counter."""
    c = np.asarray(counter, dtype=np.uint32).astype(np.uint64)
    c0, c1, c2, c3 = c[..., 0], c[..., 1], c[..., 2], c[..., 3]
    k0, k1 = int(key[0]) & 0xFFFFFFFF, int(key[1]) & 0xFFFFFFFF
    for _ in range(10):
        p0 = _MUL0 * c0   # < 2^64: exact in uint64
        p1 = _MUL1 * c2
        n0 = (p1 >> _SH) ^ c1 ^ np.uint64(k0)
        n1 = p1 & _LO
        n2 = (p0 >> _SH) ^ c3 ^ np.uint64(k1)
        n3 = p0 & _LO
        c0, c1, c2, c3 = n0, n1, n2, n3
        k0 = (k0 + _WEYL0) & 0xFFFFFFFF
        k1 = (k1 + _WEYL1) & 0xFFFFFFFF
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)
