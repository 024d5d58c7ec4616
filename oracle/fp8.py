"""8-bit floating-point codes E4M3 and E5M2 (TEST INFRASTRUCTURE ONLY).

Definition: the OCP 8-bit floating point formats (OFP8, Open Compute
Project "OCP 8-bit Floating Point Specification"): one sign bit, then

  E4M3: 4 exponent bits (bias 7), 3 mantissa bits; no infinities; the only
        NaN patterns are S.1111.111; largest finite magnitude 448 (0x7E);
        exponent field 0 holds subnormals m 2^-9.
  E5M2: 5 exponent bits (bias 15), 2 mantissa bits; exponent field 31
        holds infinities and NaNs; largest finite 57344 (0x7B); exponent
        field 0 holds subnormals m 2^-16.

Encoding used here (the optimizer state only ever encodes finite values):
round to nearest, ties to the even code (mantissa LSB 0), saturating to the
largest finite magnitude; NaN and infinity are never produced.

Pinned by torch's float8_e4m3fn / float8_e5m2 conversions (decoding of every
code; encoding of values inside the finite range, where torch rounds to
nearest even) and by the formats' landmark values.
"""

import numpy as np

# (exponent bits, mantissa bits, bias, largest finite code magnitude)
E4M3 = (4, 3, 7, 0x7E)
E5M2 = (5, 2, 15, 0x7B)


def _decode_mag(code, fmt):
    eb, mb, bias, _ = fmt
    e = (code >> mb) & ((1 << eb) - 1)
    m = code & ((1 << mb) - 1)
    sub = m.astype(np.float64) * 2.0 ** (1 - bias - mb)
    nrm = (1.0 + m.astype(np.float64) / (1 << mb)) * np.exp2(e.astype(np.float64) - bias)
    return np.where(e == 0, sub, nrm)


def decode(codes, fmt):
    """uint8 codes -> float32 values (finite codes only)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    mag = _decode_mag(c & 0x7F, fmt)
    return np.where(c & 0x80, -mag, mag).astype(np.float32)


def max_finite(fmt):
    return float(_decode_mag(np.array([fmt[3]]), fmt)[0])


def encode(x, fmt):
    """float32 values -> uint8 codes: nearest, ties to even, saturating."""
    eb, mb, bias, cmax = fmt
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x).astype(np.float64)            # exact
    sign = np.signbit(x).astype(np.int64) << 7
    top = max_finite(fmt)
    min_normal = 2.0 ** (1 - bias)
    # normal range: a = 2^e (1 + f), f in [0, 1); q = rint(f 2^mb), a carry
    # into the next binade is the next code
    safe = np.where(a > 0, a, 1.0)
    e = np.floor(np.log2(safe)).astype(np.int64)
    # log2 of a float may land one off at a binade edge: fix it exactly
    e = np.where(np.exp2(e.astype(np.float64)) > safe, e - 1, e)
    e = np.where(np.exp2((e + 1).astype(np.float64)) <= safe, e + 1, e)
    frac = safe / np.exp2(e.astype(np.float64)) - 1.0          # exact
    q = np.rint(frac * (1 << mb)).astype(np.int64)             # half to even
    normal = ((e + bias) << mb) + q
    # subnormal range: q = rint(a / 2^(1 - bias - mb))
    sub = np.rint(np.minimum(a, min_normal) / 2.0 ** (1 - bias - mb)).astype(np.int64)
    mag = np.where(a < min_normal, sub, normal)
    mag = np.where(a >= top, cmax, np.minimum(mag, cmax))
    return (mag | sign).astype(np.uint8)
