"""Adapter merge: the trained adapter folded into a 16-bit copy of the frozen
weight (TEST INFRASTRUCTURE ONLY).

Definition ([P4] "How it works", Step 8: save and use, the option that
dequantizes the base to 16 bits and merges the adapter; [P4] "Merging after
QLoRA"). With the adapter in row-vector orientation (A is [K x r], B is
[r x N], s = alpha / r) a forward pass computes

    X W'^T + s (X A) B  =  X (W' + s (A B)^T)^T,

so the merged weight is  W_m[n][k] = w'[n][k] + s * sum_j A[k][j] B[j][n],
stored in 16 bits (bfloat16, the compute type of the method).

The pages fix neither the precision nor the order of this sum. Reading
taken (the plainest one that keeps the result a deterministic function of
the inputs): w' is the float32 dequantized weight; the sum over j runs in
float32 from j = 0 upward, each product of two bfloat16 values being exact in
float32; then fl32(s * sum), fl32(w' + that), and one round-to-nearest-even
to bfloat16. A float32 implementation that keeps this order matches bit for
bit.

Pinned by: A = 0 gives bf16(w') exactly (the dequantize oracle); a brute
force on small inputs that emulates each float32 rounding with exact
rational arithmetic; and the float64 value of w' + s (A B)^T within one
bfloat16 rounding plus the float32 sum's error bound.
"""

import numpy as np

from .bf16 import f32_to_bf16_bits


def merge(w_dequant, A, B, scale):
    """Merged weight as bfloat16 bit patterns, uint16 [N x K].

    w_dequant: float32 [N x K] (the dequantized store, `dequantize`);
    A: [K x r] and B: [r x N] holding bfloat16 values (any float dtype)."""
    w = np.asarray(w_dequant, dtype=np.float32)
    A32 = np.asarray(A, dtype=np.float32)
    B32 = np.asarray(B, dtype=np.float32)
    N, K = w.shape
    r = A32.shape[1]
    assert A32.shape == (K, r) and B32.shape == (r, N)
    acc = np.zeros((N, K), dtype=np.float32)
    for j in range(r):
        # products of two bfloat16 values are exact in float32
        acc = (acc + np.outer(B32[j], A32[:, j]).astype(np.float32)).astype(np.float32)
    t = (np.float32(scale) * acc).astype(np.float32)
    m = (w + t).astype(np.float32)
    return f32_to_bf16_bits(m).reshape(N, K)
