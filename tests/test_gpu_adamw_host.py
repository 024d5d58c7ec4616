"""AdamW with its optimizer state in pinned host memory (the host-resident
half of the paged optimizer: ozercemkelahmet.com "QLoRA", How it works,
Step 7). The moments (float32 m, v; or the 8-bit codes and their scales)
live in hipHostMalloc memory mapped into the device's address space, and
the same kernels read and write them over the host link. Checked bit for
bit against the oracle over several steps, and against the same steps with
device-resident state; the pointers are confirmed to be host memory with a
device mapping before any launch."""

import ctypes

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


def _assert_mapped_host(t):
    """The tensor is pinned host memory with a device address (checked with
    hipPointerGetAttributes before the kernels touch it)."""
    assert not t.is_cuda and t.is_pinned()
    hip = ctypes.CDLL("libamdhip64.so")
    dptr = ctypes.c_void_p()
    hip.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p,
                                            ctypes.c_uint]
    assert hip.hipHostGetDevicePointer(ctypes.byref(dptr), ctypes.c_void_p(t.data_ptr()), 0) == 0
    assert dptr.value


@pytest.mark.parametrize("n", [4096, 2800, 1001, 1 << 20])
def test_adamw_host_state_bit_exact(q, n):
    print(f"[case] adamw host state n={n}", flush=True)
    dev = device()
    rng = np.random.default_rng(100 + n)
    p0 = (rng.standard_normal(n) * 0.01).astype(np.float32)
    p = torch.from_numpy(p0).to(dev)
    pd = p.clone()
    m, v = q.adamw_state(n, dev, host=True)
    md, vd = q.adamw_state(n, dev)
    for t in (m, v):
        _assert_mapped_host(t)
    p16 = torch.empty(n, dtype=torch.bfloat16, device=dev)
    hp, hm, hv = p0, np.zeros(n, np.float32), np.zeros(n, np.float32)
    for t in range(1, 4):
        gh = (rng.standard_normal(n) * 1e-3).astype(np.float32)
        g = torch.from_numpy(gh).to(dev)
        q.qlora_adamw_step(p, m, v, g, step=t, p_bf16=p16, **HP)
        q.qlora_adamw_step(pd, md, vd, g, step=t, **HP)
        hp, hm, hv = oracle.adamw_step(hp, hm, hv, gh, step=t, **HP)
        torch.cuda.synchronize()
        for name, got, want in (("p", _np(p), hp), ("m", m.numpy(), hm), ("v", v.numpy(), hv)):
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (name, t)
        assert torch.equal(p, pd) and torch.equal(m, md.cpu()) and torch.equal(v, vd.cpu())
        got16 = _np(p16.view(torch.int16)).view(np.uint16)
        assert np.array_equal(got16, f32_to_bf16_bits(hp)), ("bf16", t)


@pytest.mark.parametrize("n", [4096, 1001, 1 << 20])
def test_adamw8_host_state_bit_exact(q, n):
    print(f"[case] adamw8 host state n={n}", flush=True)
    dev = device()
    rng = np.random.default_rng(200 + n)
    p0 = (rng.standard_normal(n) * 0.01).astype(np.float32)
    p = torch.from_numpy(p0).to(dev)
    pd = p.clone()
    m8, sm, v8, sv = q.adamw8_state(n, dev, host=True)
    dm8, dsm, dv8, dsv = q.adamw8_state(n, dev)
    for t in (m8, sm, v8, sv):
        _assert_mapped_host(t)
    nb = oracle.num_blocks8(n)
    hp = p0
    hm8 = np.zeros(n, np.uint8); hv8 = np.zeros(n, np.uint8)
    hsm = np.zeros(nb, np.float32); hsv = np.zeros(nb, np.float32)
    for t in range(1, 5):
        # gradients over several decades, so that the codes span their range
        gh = (rng.standard_normal(n) * 10.0 ** rng.uniform(-6, -2, n)).astype(np.float32)
        g = torch.from_numpy(gh).to(dev)
        q.qlora_adamw8_step(p, m8, sm, v8, sv, g, step=t, **HP)
        q.qlora_adamw8_step(pd, dm8, dsm, dv8, dsv, g, step=t, **HP)
        hp, hm8, hsm, hv8, hsv = oracle.adamw8_step(hp, hm8, hsm, hv8, hsv, gh, step=t, **HP)
        torch.cuda.synchronize()
        assert np.array_equal(_np(p).view(np.uint32), hp.view(np.uint32)), ("p", t)
        assert np.array_equal(m8.numpy(), hm8) and np.array_equal(v8.numpy(), hv8), t
        assert np.array_equal(sm.numpy().view(np.uint32), hsm.view(np.uint32)), ("sm", t)
        assert np.array_equal(sv.numpy().view(np.uint32), hsv.view(np.uint32)), ("sv", t)
        for a, b in ((m8, dm8), (sm, dsm), (v8, dv8), (sv, dsv)):
            assert torch.equal(a, b.cpu())


def test_host_state_must_be_pinned(q):
    """Pageable host memory is refused by the binding before any launch."""
    dev = device()
    n = 1024
    p = torch.zeros(n, device=dev)
    g = torch.zeros(n, device=dev)
    m = torch.zeros(n)  # pageable
    v = torch.zeros(n, pin_memory=True)
    with pytest.raises(q.QloraError):
        q.qlora_adamw_step(p, m, v, g, 1e-3, step=1)
