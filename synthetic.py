"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no arithmetic of the method: it only draws random tensors
and names the workload shapes. Every tensor is drawn in float32 from its own
torch.Generator, seeded with  seed * 1_000_003 + index  (index fixed per
tensor role and layer), then rounded to bfloat16 (round to nearest even).

Distributions (standard deviations, not variances):
  weights      N(0, 0.02), or Student-t with 5 degrees of freedom times 0.02
               for the heavy-tailed 65B-shaped stress case
  activations  N(0, 1);  upstream gradients N(0, 1e-3)
  adapters     A, B ~ N(0, 0.01)
The weight shapes are LLaMA-style decoder linears (q, k, v, o, gate, up,
down); models, checkpoints and datasets are not used.
"""

import torch

# role indices inside one linear's draw
W_IDX, X_IDX, A_IDX, B_IDX, DY_IDX = 0, 1, 2, 3, 4


def _gen(device, seed, index):
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1_000_003 + index)
    return g


def normal(shape, std, device, seed, index):
    g = _gen(device, seed, index)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return (x * std).to(torch.bfloat16)


def student_t(shape, df, scale, device, seed, index):
    """t = Z / sqrt(chi2_df / df) with chi2_df a sum of df squared normals."""
    g = _gen(device, seed, index)
    z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    chi = torch.zeros(shape, device=device, dtype=torch.float32)
    for _ in range(int(df)):
        e = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        chi.addcmul_(e, e)
    return (z / torch.sqrt(chi / df) * scale).to(torch.bfloat16)


def linear_inputs(M, N, K, r, device, seed=0, base=0, weight="normal", need_dy=True):
    """W [N x K], X [M x K], A [K x r], B [r x N], dY [M x N] for one linear.

    `base` offsets the generator indices so that distinct linears (layers,
    projections) draw independent tensors."""
    if weight == "normal":
        W = normal((N, K), 0.02, device, seed, base + W_IDX)
    elif weight == "student_t":
        W = student_t((N, K), 5, 0.02, device, seed, base + W_IDX)
    else:
        raise ValueError(weight)
    X = normal((M, K), 1.0, device, seed, base + X_IDX)
    A = normal((K, r), 0.01, device, seed, base + A_IDX)
    B = normal((r, N), 0.01, device, seed, base + B_IDX)
    dY = normal((M, N), 1e-3, device, seed, base + DY_IDX) if need_dy else None
    return W, X, A, B, dY


# The five workloads: (name, linears [(N, K)], M list, r, alpha, layers, weight dist)
LLAMA7B = [(4096, 4096)] * 4 + [(11008, 4096)] * 2 + [(4096, 11008)]
LLAMA65B = [(8192, 8192)] * 4 + [(22016, 8192)] * 2 + [(8192, 22016)]

WORKLOADS = {
    "single_256": dict(linears=[(256, 256)], M=[16], r=8, alpha=16, layers=1,
                       weight="normal", bwd=True),
    "decode_gemv_4096": dict(linears=[(4096, 4096)], M=[1, 4, 16], r=16, alpha=32, layers=1,
                             weight="normal", bwd=False),
    "prefill_mlp_7b": dict(linears=[(11008, 4096), (11008, 4096), (4096, 11008)], M=[2048],
                           r=64, alpha=16, layers=1, weight="normal", bwd=True),
    "stack_7b": dict(linears=LLAMA7B, M=[2048], r=64, alpha=16, layers=32, weight="normal",
                     bwd=True),
    "stress_65b": dict(linears=LLAMA65B, M=[4096], r=64, alpha=16, layers=80,
                       weight="student_t", bwd=True),
}


def linear_base(layer, j):
    """Generator index base of linear j of layer `layer` (5 tensors each)."""
    return (layer * 16 + j) * 8
