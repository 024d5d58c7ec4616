"""Pins of the adapter-merge oracle (oracle.merge) against facts outside it:
the dequantize oracle for a zero adapter, a brute force that emulates every
float32 rounding with exact rational arithmetic, and the float64 value within
the rounding bound."""

from fractions import Fraction
import struct

import numpy as np
import pytest

import oracle


def _round_sig(x, p):
    """Round a rational to p significant bits, ties to even (no exponent
    limits: the values here are far from float32's range ends)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    x = abs(x)
    e = x.numerator.bit_length() - x.denominator.bit_length()
    while Fraction(2) ** e > x:
        e -= 1
    while Fraction(2) ** (e + 1) <= x:
        e += 1
    ulp = Fraction(2) ** (e - (p - 1))
    q = x / ulp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def _bf16_bits(x):
    """Bit pattern of a rational that is exactly a bfloat16 value."""
    b = struct.unpack("<I", struct.pack("<f", float(x)))[0]
    assert b & 0xFFFF == 0
    return b >> 16


def _store(N, K, seed):
    rng = np.random.default_rng(seed)
    w = oracle.bf16_round((rng.standard_normal(N * K) * 0.02).astype(np.float32))
    st = oracle.quantize(w)
    return oracle.dequantize(st["codes"], st["absmax_q"], st["absmax_s2"], N * K).reshape(N, K)


def _bf16_values(shape, scale, seed):
    rng = np.random.default_rng(seed)
    return oracle.bf16_round((rng.standard_normal(shape) * scale).astype(np.float32))


def test_zero_adapter_is_dequantized_weight():
    N, K, r = 64, 128, 8
    wp = _store(N, K, 1)
    A = np.zeros((K, r), np.float32)
    B = _bf16_values((r, N), 0.01, 2)
    got = oracle.merge(wp, A, B, 0.25)
    assert np.array_equal(got, oracle.f32_to_bf16_bits(wp).reshape(N, K))


@pytest.mark.parametrize("scale", [0.25, 0.37])
def test_brute_force_rational(scale):
    """Every float32 rounding of the definition emulated exactly."""
    N, K, r = 3, 64, 5
    wp = _store(N, K, 3)
    A = _bf16_values((K, r), 0.5, 4)
    B = _bf16_values((r, N), 0.5, 5)
    got = oracle.merge(wp, A, B, scale)
    s = Fraction(float(np.float32(scale)))
    for n in range(N):
        for k in range(K):
            acc = Fraction(0)
            for j in range(r):
                acc = _round_sig(acc + Fraction(float(A[k, j])) * Fraction(float(B[j, n])), 24)
            t = _round_sig(s * acc, 24)
            m = _round_sig(Fraction(float(wp[n, k])) + t, 24)
            assert got[n, k] == _bf16_bits(_round_sig(m, 8)), (n, k)


def test_float64_value_within_rounding_bound():
    N, K, r, s = 128, 256, 16, 0.25
    wp = _store(N, K, 6)
    A = _bf16_values((K, r), 0.01, 7)
    B = _bf16_values((r, N), 0.01, 8)
    got = oracle.bf16_bits_to_f32(oracle.merge(wp, A, B, s)).reshape(N, K).astype(np.float64)
    exact = wp.astype(np.float64) + s * (A.astype(np.float64) @ B.astype(np.float64)).T
    absprod = s * (np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64))).T
    # bfloat16 rounding (half an ulp: 2^-8 relative) of a float32 value whose
    # own error is at most r float32 roundings of the sum plus two more
    bound = 2.0 ** -8 * np.abs(exact) * 1.001 + (r + 2) * 2.0 ** -24 * (absprod + np.abs(wp)) * 2
    assert np.all(np.abs(got - exact) <= bound + 1e-30)
    # and the adapter term is visible: the merge differs from bf16(w') somewhere
    assert np.any(got != oracle.bf16_round(wp).astype(np.float64))
