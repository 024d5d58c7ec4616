"""Pins for the oracle's 8-bit floating-point codes and the AdamW step with
8-bit state (CPU only).

  * E4M3 / E5M2 decoding of every code, and encoding of random values, of
    every midpoint between neighbouring codes and of the values one float32
    step either side of them, against torch's float8_e4m3fn / float8_e5m2
    conversions; the formats' landmark values; saturation;
  * the 8-bit step: the block maximum of each new moment encodes to the
    largest finite code; decoded moments lie within half a code step of the
    float32 moments; the first step from a zero state equals the float32
    AdamW (the decoded zero state is exact); blocks are independent; a zero
    gradient and a zero state leave p to the decoupled decay alone;
  * a planted mistake (a linear 8-bit code for v) fails the half-step bound.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8

FMTS = [(fp8.E4M3, torch.float8_e4m3fn, 448.0), (fp8.E5M2, torch.float8_e5m2, 57344.0)]


@pytest.mark.parametrize("fmt,tdt,top", FMTS)
def test_decode_every_code(fmt, tdt, top):
    codes = np.arange(256, dtype=np.uint8)
    ours = fp8.decode(codes, fmt)
    theirs = torch.from_numpy(codes.copy()).view(tdt).float().numpy()
    finite = np.isfinite(theirs)
    assert np.array_equal(ours[finite].view(np.uint32), theirs[finite].view(np.uint32))
    assert fp8.max_finite(fmt) == top


def test_landmarks():
    assert fp8.decode(np.array([0x7E, 0x08, 0x01, 0x38], np.uint8), fp8.E4M3).tolist() == \
        [448.0, 2.0 ** -6, 2.0 ** -9, 1.0]
    assert fp8.decode(np.array([0x7B, 0x04, 0x01, 0x3C], np.uint8), fp8.E5M2).tolist() == \
        [57344.0, 2.0 ** -14, 2.0 ** -16, 1.0]


@pytest.mark.parametrize("fmt,tdt,top", FMTS)
def test_encode_against_torch(fmt, tdt, top):
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(500_000) * np.exp(rng.uniform(-30, 12, 500_000))).astype(np.float32)
    x = x[np.abs(x) <= top]
    # every midpoint between neighbouring finite values, and one float32 step
    # either side of it
    pos = np.arange(0, fmt[3] + 1, dtype=np.uint8)
    vals = fp8.decode(pos, fmt).astype(np.float64)
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    near = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(np.inf))])
    x = np.concatenate([x, near, -near, vals.astype(np.float32), -vals.astype(np.float32)])
    ours = fp8.encode(x, fmt)
    theirs = torch.from_numpy(x).to(tdt).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


@pytest.mark.parametrize("fmt,top", [(fp8.E4M3, 448.0), (fp8.E5M2, 57344.0)])
def test_encode_saturates(fmt, top):
    x = np.array([top, top * 1.01, 1e30, -1e30], np.float32)
    assert fp8.encode(x, fmt).tolist() == [fmt[3], fmt[3], fmt[3], fmt[3] | 0x80]


def _state(n, seed):
    rng = np.random.default_rng(seed)
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    gs = [(rng.standard_normal(n) * np.exp(rng.uniform(-6, 0, n)) * 1e-3).astype(np.float32)
          for _ in range(4)]
    return p, gs


def _run8(p, gs, wd=0.01):
    n = p.size
    nb = oracle.num_blocks8(n)
    m8 = np.zeros(n, np.uint8); v8 = np.zeros(n, np.uint8)
    sm = np.zeros(nb, np.float32); sv = np.zeros(nb, np.float32)
    out = []
    for t, g in enumerate(gs, start=1):
        p, m8, sm, v8, sv = oracle.adamw8_step(p, m8, sm, v8, sv, g, 2e-4, 0.9, 0.999, 1e-8, wd, t)
        out.append((p, m8, sm, v8, sv))
    return out


def test_block_max_encodes_to_top_code():
    p, gs = _state(256 * 5 + 17, 2)
    for p1, m8, sm, v8, sv in _run8(p, gs):
        for b in range(oracle.num_blocks8(p.size)):
            sl = slice(b * 256, (b + 1) * 256)
            assert np.max(m8[sl] & 0x7F) == 0x7E
            assert np.max(v8[sl]) == 0x7B


def test_decoded_moments_within_half_step():
    p, gs = _state(256 * 8, 3)
    n = p.size
    m = np.zeros(n, np.float32); v = np.zeros(n, np.float32)
    nb = n // 256
    m8 = np.zeros(n, np.uint8); v8 = np.zeros(n, np.uint8)
    sm = np.zeros(nb, np.float32); sv = np.zeros(nb, np.float32)
    for t, g in enumerate(gs, start=1):
        # the float32 moments that the 8-bit step quantizes
        md = oracle.dequantize_state(m8, sm, fp8.E4M3)
        vd = oracle.dequantize_state(v8, sv, fp8.E5M2)
        _, m1, v1 = oracle.adamw_step(p, md, vd, g, 2e-4, 0.9, 0.999, 1e-8, 0.0, t)
        p, m8, sm, v8, sv = oracle.adamw8_step(p, m8, sm, v8, sv, g, 2e-4, 0.9, 0.999, 1e-8, 0.0, t)
        mq = oracle.dequantize_state(m8, sm, fp8.E4M3).astype(np.float64)
        vq = oracle.dequantize_state(v8, sv, fp8.E5M2).astype(np.float64)
        blk = np.arange(n) // 256
        # relative half step 2^-4 (E4M3) / 2^-3 (E5M2) for normal codes, an
        # absolute half step of the smallest subnormal below them
        tol_m = np.maximum(np.abs(m1) * 2.0 ** -4, sm[blk] * 2.0 ** -10) * (1 + 1e-6)
        tol_v = np.maximum(np.abs(v1) * 2.0 ** -3, sv[blk] * 2.0 ** -17) * (1 + 1e-6)
        assert np.all(np.abs(mq - m1) <= tol_m)
        assert np.all(np.abs(vq - v1) <= tol_v)


def test_first_step_equals_float32():
    p, gs = _state(1000, 4)
    p1 = _run8(p, gs[:1])[0][0]
    want, _, _ = oracle.adamw_step(p, np.zeros_like(p), np.zeros_like(p), gs[0], 2e-4, 0.9, 0.999,
                                   1e-8, 0.01, 1)
    assert np.array_equal(p1.view(np.uint32), want.view(np.uint32))


def test_blocks_independent():
    p, gs = _state(256 * 3, 5)
    a = _run8(p, gs)
    gs2 = [g.copy() for g in gs]
    for g in gs2:
        g[256:512] *= 100.0
    b = _run8(p, gs2)
    for (pa, ma, sa, va, wa), (pb, mb, sb, vb, wb) in zip(a, b):
        for sl in (slice(0, 256), slice(512, 768)):
            assert np.array_equal(pa[sl], pb[sl]) and np.array_equal(ma[sl], mb[sl])
            assert np.array_equal(va[sl], vb[sl])
        assert sa[0] == sb[0] and sa[2] == sb[2] and sa[1] != sb[1]


def test_zero_gradient_is_pure_decay():
    p, _ = _state(700, 6)
    gs = [np.zeros_like(p)] * 3
    q = p.copy()
    lw = np.float32(np.float32(2e-4) * np.float32(0.05))
    for (p1, m8, sm, v8, sv) in _run8(p, gs, wd=0.05):
        q = (q - (lw * q).astype(np.float32)).astype(np.float32)
        assert np.array_equal(p1.view(np.uint32), q.view(np.uint32))
        assert not m8.any() and not v8.any() and not sm.any() and not sv.any()


def test_planted_linear_code_fails_bound():
    """A linear 8-bit code for v, scaled by the block maximum, loses the
    small second moments that the E5M2 code keeps."""
    rng = np.random.default_rng(7)
    v = (np.exp(rng.uniform(-20, 0, 256)) * 1e-6).astype(np.float32)
    amax = np.float32(v.max())
    lin = np.rint(v / amax * np.float32(255)) * (amax / np.float32(255))
    assert np.any(np.abs(lin - v) > np.abs(v) * 2.0 ** -3 + amax * 2.0 ** -17 / 57344)
    codes, scale = oracle.quantize_state(v, fp8.E5M2, 57344.0)
    back = oracle.dequantize_state(codes, scale, fp8.E5M2)
    assert np.all(np.abs(back - v) <= np.maximum(np.abs(v) * 2.0 ** -3, scale[0] * 2.0 ** -17) * (1 + 1e-6))
