"""Forward and backward of the frozen NF4 linear layer with a LoRA term.

TEST INFRASTRUCTURE ONLY.

Definition ([P4] "Step 5: forward pass with on-the-fly dequantization" and
"Step 6: backward pass"; [P2] "Training Flow"; [P5] "The crucial split:
store in four bits, compute in sixteen"):

  the stored weight is dequantized and rounded to the bfloat16 compute type,
  W' = bf16(w'), and with the adapter in row-vector orientation
  (A is [K x r], B is [r x N], s = alpha / r),

      T  = X A                       [M x r]
      Y  = X W'^T + s T B            [M x N]

  and for an upstream gradient dY, gradients reach only the adapter and the
  input; the frozen 4-bit weight gets none:

      G  = dY B^T                    [M x r]
      dX = dY W' + s G A^T           [M x K]
      dA = s X^T G                   [K x r]
      dB = s T^T dY                  [r x N]

The pages write the adapter in column form, (alpha/r) B (A x); the row form
above is its transpose and is what a [tokens x features] activation needs.

All products are of exact bfloat16 values and are accumulated in float64
(no rounding of T, G or of any partial sum), so the oracle is at least as
accurate as any float32-accumulating implementation.

With LoRA dropout (oracle.dropout) the adapter path takes D(X) in place
of X, and the chain rule sends its input gradient back through the same mask
and scale.

Pinned against torch.autograd in float64 on the dense weight (with and
without a dropout mask), against finite differences, and by exact special
cases (B = 0, A = 0, s = 0, W' = 0, an all-ones mask with scale 1).
"""

import numpy as np

from .bf16 import bf16_round


def _f64(a):
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def _dropped(X, keep, keep_scale):
    """D(X) = (X o keep) keep_scale, the adapter's input (oracle.dropout)."""
    if keep is None:
        return X
    return np.where(np.asarray(keep, dtype=bool), X, 0.0) * float(keep_scale)


def linear_fwd(X, w_dequant, A, B, scale, keep=None, keep_scale=1.0):
    """Returns (Y, T) in float64. X, A, B hold bfloat16-exact values;
    w_dequant is the float32 [N x K] output of `dequantize`. With a dropout
    mask `keep` (bool [M x K]), the adapter path takes D(X) instead of X and
    T = D(X) A."""
    X = _f64(X)
    Wb = _f64(bf16_round(np.asarray(w_dequant, dtype=np.float32)))
    A = _f64(A)
    B = _f64(B)
    T = _dropped(X, keep, keep_scale) @ A
    Y = X @ Wb.T + float(scale) * (T @ B)
    return Y, T


def linear_bwd(dY, X, w_dequant, A, B, scale, keep=None, keep_scale=1.0):
    """Returns (dX, dA, dB) in float64. With a dropout mask the adapter
    path's input gradient passes through the same mask and scale:
    dX = dY W' + s ((G A^T) o keep) keep_scale, dA = s D(X)^T G,
    dB = s T^T dY with T = D(X) A."""
    dY = _f64(dY)
    X = _f64(X)
    Wb = _f64(bf16_round(np.asarray(w_dequant, dtype=np.float32)))
    A = _f64(A)
    B = _f64(B)
    s = float(scale)
    Xd = _dropped(X, keep, keep_scale)
    T = Xd @ A
    G = dY @ B.T
    dX = dY @ Wb + s * _dropped(G @ A.T, keep, keep_scale)
    dA = s * (Xd.T @ G)
    dB = s * (T.T @ dY)
    return dX, dA, dB
