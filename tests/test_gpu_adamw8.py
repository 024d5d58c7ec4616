"""GPU AdamW step with 8-bit state (qlora_adamw8_step) against the oracle,
bit for bit over successive steps: parameters, both code arrays, both scale
arrays and the bf16 copy; the vector path, the scalar path (shifted
pointers), a short last block, a single short block, gradients spanning
many decades (subnormal codes) and a full-size adapter set on sampled
blocks (blocks are independent, so a block's oracle run is exact)."""

import numpy as np
import pytest
import torch

import oracle
from oracle.bf16 import f32_to_bf16_bits
from tests.gpu_util import device

pytestmark = pytest.mark.gpu

HP = dict(lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


@pytest.fixture(scope="module")
def q():
    device()
    import bit_quantized_finetuning_quantize_amd as q
    return q


def _np(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _grad(rng, n, decades):
    return (rng.standard_normal(n) * np.exp(rng.uniform(-decades * 2.3, 0, n)) * 1e-3).astype(np.float32)


@pytest.mark.parametrize("n,shift,decades", [(256 * 7, 0, 1), (1001, 0, 3), (4097, 1, 2),
                                             (255, 3, 6), (256 * 40, 0, 8)])
def test_adamw8_bit_exact_over_steps(q, n, shift, decades):
    print(f"[case] adamw8 n={n} shift={shift} decades={decades}", flush=True)
    dev = device()
    rng = np.random.default_rng(n + shift)
    nb = oracle.num_blocks8(n)
    p0 = (rng.standard_normal(n) * 0.01).astype(np.float32)
    fbuf = {k: torch.zeros(n + shift, dtype=torch.float32, device=dev) for k in "pg"}
    p, g = fbuf["p"][shift:], fbuf["g"][shift:]
    cbuf = {k: torch.zeros(n + shift, dtype=torch.uint8, device=dev) for k in "mv"}
    m8, v8 = cbuf["m"][shift:], cbuf["v"][shift:]
    sm = torch.zeros(nb, dtype=torch.float32, device=dev)
    sv = torch.zeros(nb, dtype=torch.float32, device=dev)
    p.copy_(torch.from_numpy(p0))
    p16 = torch.empty(n, dtype=torch.bfloat16, device=dev)
    hp = p0
    hm8, hv8 = np.zeros(n, np.uint8), np.zeros(n, np.uint8)
    hsm, hsv = np.zeros(nb, np.float32), np.zeros(nb, np.float32)
    for t in range(1, 5):
        gh = _grad(rng, n, decades)
        g.copy_(torch.from_numpy(gh))
        q.qlora_adamw8_step(p, m8, sm, v8, sv, g, step=t, p_bf16=p16, **HP)
        hp, hm8, hsm, hv8, hsv = oracle.adamw8_step(hp, hm8, hsm, hv8, hsv, gh, step=t, **HP)
        assert np.array_equal(_np(p).view(np.uint32), hp.view(np.uint32)), ("p", t)
        assert np.array_equal(_np(m8), hm8), ("m8", t)
        assert np.array_equal(_np(v8), hv8), ("v8", t)
        assert np.array_equal(_np(sm).view(np.uint32), hsm.view(np.uint32)), ("sm", t)
        assert np.array_equal(_np(sv).view(np.uint32), hsv.view(np.uint32)), ("sv", t)
        got16 = _np(p16.view(torch.int16)).view(np.uint16)
        assert np.array_equal(got16, f32_to_bf16_bits(hp)), ("bf16", t)


def test_adamw8_full_adapter_set(q):
    """All adapters of the 32-layer 7B-style stack at r = 64 (159,907,840
    parameters), two steps; 300 sampled blocks against the oracle."""
    dev = device()
    n = 32 * 64 * (4 * (4096 + 4096) + 2 * (4096 + 11008) + (11008 + 4096))
    nb = oracle.num_blocks8(n)
    print(f"[case] adamw8 n={n}", flush=True)
    gen = torch.Generator(device=dev).manual_seed(9)
    p = torch.randn(n, device=dev, generator=gen) * 0.01
    m8, sm, v8, sv = q.adamw8_state(n, dev)
    blocks = np.sort(np.random.default_rng(1).choice(nb, 300, replace=False))
    idx = torch.from_numpy((blocks[:, None] * 256 + np.arange(256)).ravel()).to(dev)
    hp = _np(p[idx])
    hm8 = np.zeros(idx.numel(), np.uint8); hv8 = np.zeros(idx.numel(), np.uint8)
    hsm = np.zeros(300, np.float32); hsv = np.zeros(300, np.float32)
    for t in (1, 2):
        g = torch.randn(n, device=dev, generator=gen) * 1e-3
        gh = _np(g[idx])
        q.qlora_adamw8_step(p, m8, sm, v8, sv, g, step=t, **HP)
        hp, hm8, hsm, hv8, hsv = oracle.adamw8_step(hp, hm8, hsm, hv8, hsv, gh, step=t, **HP)
        del g
    bi = torch.from_numpy(blocks).to(dev)
    assert np.array_equal(_np(p[idx]).view(np.uint32), hp.view(np.uint32))
    assert np.array_equal(_np(m8[idx]), hm8) and np.array_equal(_np(v8[idx]), hv8)
    assert np.array_equal(_np(sm[bi]).view(np.uint32), hsm.view(np.uint32))
    assert np.array_equal(_np(sv[bi]).view(np.uint32), hsv.view(np.uint32))
