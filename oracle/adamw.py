"""AdamW step for the adapter parameters, float32 state (TEST INFRASTRUCTURE
ONLY).

The pages name AdamW with 32-bit or 8-bit state, paged, as the optimizer of
the trained adapters ([P4] "Practical guidance and best practices",
Optimizer and schedule; [P4] "How it works", Step 7) and do not restate it.
AdamW is Adam's bias-corrected moment estimates with a weight decay that is
decoupled from the gradient (Loshchilov and Hutter, "Decoupled Weight Decay
Regularization"). Reading taken for the float32 variant: every operation is
one float32 operation rounded on its own, in the order

    lw = fl(lr wd),  ob1 = fl(1 - b1),  ob2 = fl(1 - b2)      (host, float64
    c1 = fl(1 - b1^t),  c2 = fl(1 - b2^t)                     then rounded)
    p1 = p - lw p
    m  = b1 m + ob1 g
    v  = b2 v + ob2 (g g)
    p  = p1 - lr ((m / c1) / (sqrt(v / c2) + eps))

with correctly rounded division and square root, so a float32 implementation
in this order matches bit for bit.

Pinned by torch.optim.AdamW in float64 over several steps (within the float32
rounding of each step), the zero-gradient closed form (pure decoupled
decay, exact), and the first-step closed form (|update| <= lr).
"""

import numpy as np


def adamw_step(p, m, v, g, lr, beta1, beta2, eps, weight_decay, step):
    """Return (p, m, v) after one step; inputs float32 arrays (not modified)."""
    f = np.float32
    p = np.asarray(p, dtype=f)
    m = np.asarray(m, dtype=f)
    v = np.asarray(v, dtype=f)
    g = np.asarray(g, dtype=f)
    lr32, b1, b2, eps32 = f(lr), f(beta1), f(beta2), f(eps)
    lw = f(float(lr32) * float(f(weight_decay)))
    ob1 = f(1.0 - float(b1))
    ob2 = f(1.0 - float(b2))
    c1 = f(1.0 - float(b1) ** int(step))
    c2 = f(1.0 - float(b2) ** int(step))
    p1 = (p - (lw * p).astype(f)).astype(f)
    m1 = ((b1 * m).astype(f) + (ob1 * g).astype(f)).astype(f)
    v1 = ((b2 * v).astype(f) + (ob2 * (g * g).astype(f)).astype(f)).astype(f)
    den = (np.sqrt((v1 / c2).astype(f)).astype(f) + eps32).astype(f)
    upd = (lr32 * ((m1 / c1).astype(f) / den).astype(f)).astype(f)
    return (p1 - upd).astype(f), m1, v1
