"""Pins of the AdamW oracle (oracle.adamw_step): torch.optim.AdamW in float64,
the zero-gradient closed form (pure decoupled decay) and the first-step
bound."""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

HP = dict(lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def _rand(n, seed, scale):
    return (np.random.default_rng(seed).standard_normal(n) * scale).astype(np.float32)


def test_matches_torch_adamw_float64_over_steps():
    n = 4096
    p = _rand(n, 0, 0.01)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    tp = torch.tensor(p, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([tp], lr=HP["lr"], betas=(HP["beta1"], HP["beta2"]), eps=HP["eps"],
                            weight_decay=HP["weight_decay"])
    for t in range(1, 6):
        g = _rand(n, 10 + t, 1e-3)
        p, m, v = oracle.adamw_step(p, m, v, g, step=t, **HP)
        tp.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        ref = tp.detach().numpy()
        # the float32 roundings of each step (a few ulps of p per step) and a
        # relative 1e-4 of the step size for the rounded update itself
        ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(p - ref) <= 4 * t * ulp + 1e-4 * HP["lr"] * t), t


def test_zero_gradient_is_pure_decoupled_decay():
    n = 257
    p = _rand(n, 1, 0.05)
    z = np.zeros(n, np.float32)
    p1, m1, v1 = oracle.adamw_step(p, z, z, z, step=3, **HP)
    assert not np.any(m1) and not np.any(v1)
    lw = np.float32(float(np.float32(HP["lr"])) * float(np.float32(HP["weight_decay"])))
    for i in range(n):
        # p - fl(lw p), each rounding to nearest float32 (numpy's scalar ops are
        # correctly rounded; the product and difference are checked exactly)
        prod = Fraction(float(lw)) * Fraction(float(p[i]))
        want_prod = np.float32(float(prod))  # float() of a rational rounds once to float64
        assert Fraction(float(want_prod)) - prod <= abs(prod) * Fraction(1, 2 ** 23)
        assert p1[i] == np.float32(p[i] - want_prod)


def test_first_step_moves_by_at_most_lr():
    n = 1000
    p = _rand(n, 2, 0.02)
    g = _rand(n, 3, 1.0)
    z = np.zeros(n, np.float32)
    hp = dict(HP, weight_decay=0.0)
    p1, m1, v1 = oracle.adamw_step(p, z, z, g, step=1, **hp)
    step_taken = (p1.astype(np.float64) - p) / hp["lr"]
    # first step: m/c1 = g, sqrt(v/c2) = |g| up to rounding, so each
    # coordinate moves by lr |g| / (|g| + eps), against the sign of g
    assert np.all(np.abs(step_taken) <= 1.0 + 1e-4)
    assert np.all(np.sign(step_taken[np.abs(g) > 1e-3]) == -np.sign(g[np.abs(g) > 1e-3]))
    assert np.allclose(np.abs(step_taken), 1.0, atol=1e-3)
