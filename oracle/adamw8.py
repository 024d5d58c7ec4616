"""AdamW step with 8-bit optimizer state (TEST INFRASTRUCTURE ONLY).

The pages' recipe trains the adapters with a paged 8-bit AdamW ([P4] "A code
example with common libraries", Training arguments, optim; "Practical
guidance and best practices", Optimizer and schedule: a paged 8-bit or
32-bit AdamW) and do not say how the state is held in 8 bits. Reading taken
here: the pages' own scheme for the weights -- blocks with an absmax scale --
applied to each moment, with an 8-bit floating-point code (oracle.fp8) so
that values many decades below the block maximum keep a relative precision:

  blocks of BLOCK8 = 256 consecutive parameters, one float32 scale each;
  first moment m:  E4M3 codes, scale sm = fl(max|m| / 448)
  second moment v: E5M2 codes, scale sv = fl(max v / 57344)
  code = encode(fl(x / scale)), 0 when scale = 0;  x' = fl(decode(code) scale)

(a linear 8-bit code would turn every v below 1/510 of its block maximum
into 0, and with it the update's denominator into eps).

One step, every operation one float32 operation in this order (the float32
AdamW of oracle.adamw on the decoded moments):

  m = fl(dec(m8) sm),  v = fl(dec(v8) sv)
  p1 = p - lw p,  m1 = b1 m + ob1 g,  v1 = b2 v + ob2 (g g)
  p2 = p1 - lr ((m1 / c1) / (sqrt(v1 / c2) + eps))
  sm' = fl(max_block |m1| / 448),  sv' = fl(max_block v1 / 57344)
  m8' = enc_E4M3(fl(m1 / sm')),  v8' = enc_E5M2(fl(v1 / sv'))

A short final block takes its maximum over the parameters present.

Pinned by: the block maximum encodes to the largest finite code (so the
scale definition is visible in the stored state), decoded moments within
half a code step of the float32 moments, agreement with the float32 AdamW
in the first step (where the decoded zero state is exact), blocks being
independent of each other, and the zero-gradient closed form.
"""

import numpy as np

from . import fp8
from .adamw import adamw_step

BLOCK8 = 256


def num_blocks8(n):
    return -(-int(n) // BLOCK8)


def _block_max(x):
    n = x.size
    nb = num_blocks8(n)
    pad = np.zeros(nb * BLOCK8, dtype=np.float32)
    pad[:n] = x
    return pad.reshape(nb, BLOCK8).max(axis=1)


def quantize_state(x, fmt, top):
    """float32 moment -> (codes uint8 [n], scales float32 [nblocks])."""
    f = np.float32
    x = np.asarray(x, dtype=f)
    amax = _block_max(np.abs(x))
    scale = (amax / f(top)).astype(f)
    blk = np.arange(x.size) // BLOCK8
    s = scale[blk]
    y = (x / np.where(s == 0, f(1), s)).astype(f)
    codes = fp8.encode(y, fmt)
    codes[s == 0] = 0
    return codes, scale


def dequantize_state(codes, scale, fmt):
    blk = np.arange(np.asarray(codes).size) // BLOCK8
    return (fp8.decode(codes, fmt) * np.asarray(scale, np.float32)[blk]).astype(np.float32)


def adamw8_step(p, m8, sm, v8, sv, g, lr, beta1, beta2, eps, weight_decay, step):
    """Return (p, m8, sm, v8, sv) after one step (inputs are not modified)."""
    m = dequantize_state(m8, sm, fp8.E4M3)
    v = dequantize_state(v8, sv, fp8.E5M2)
    p2, m1, v1 = adamw_step(p, m, v, g, lr, beta1, beta2, eps, weight_decay, step)
    m8n, smn = quantize_state(m1, fp8.E4M3, 448.0)
    v8n, svn = quantize_state(v1, fp8.E5M2, 57344.0)
    return p2, m8n, smn, v8n, svn
