"""NF4 blockwise quantization with double quantization (TEST INFRASTRUCTURE ONLY).

What is computed, and where the pages say so:

* Codebook. 16 NormalFloat levels placed at quantiles of the standard normal
  so that each bin carries the same probability mass, then scaled into
  [-1, 1] ([P2] "How It Works" item 1; [P4] "How it works / Why NormalFloat";
  [P5] "Three refinements that keep the intelligence intact").
  Readings where the pages are silent:
  the type keeps an exact zero and both endpoints -1 and +1, which forces an
  asymmetric split (7 negative levels, 0, 8 positive levels, equal mass per
  bin within each half); the inverse CDF at 1 is infinite, so the outermost
  probability is truncated at P_MAX = 1 - (1/30 + 1/32)/2 = 929/960.
  The construction given P_MAX is pinned by invariants (monotone, exact 0,
  endpoints +-1, equal spacing in probability per half) and by a second,
  independent inverse CDF; the value of P_MAX itself is a reading:
  parity unpinned by the pages for that one constant.

* Level-1 quantization. Consecutive runs of BLOCK = 64 values of the flat
  row-major tensor form a block; each block is divided by its largest
  absolute value and every normalized value is replaced by the index of the
  nearest level ([P4] "Step 1: quantize the base weights to 4 bits",
  "Step 2: store the scale per block", "A worked example").
  Readings: division is one IEEE float32 division w / c; nearest is exact
  distance with ties to the lower index; an all-zero block has c = 0 and
  every code is the index of level 0; a short final block takes its maximum
  over the elements present; element 2i sits in the low nibble of byte i.

* Level-2 (double) quantization. The per-block constants are themselves
  quantized from 32 bits to 8 bits in groups of GROUP = 256 constants, each
  group keeping one float32 second-level constant ([P1] "How It Works" item
  2; [P2] "How It Works" item 2; [P4] "Step 3: double quantization").
  Reading: an unsigned linear absmax code, q8 = round_half_even(255 *
  fl32(c / s2)) with s2 the group maximum (the constants are >= 0, so all
  256 codes are usable); an all-zero group stores q8 = 0, s2 = 0.
  Pinned by the 0.37-bit saving the pages state (closed form 0.373046875),
  by q8 = 255 at the group maximum and by the half-step error bound.

* Without double quantization ([P4] "Step 2: store the scale per block": a
  32-bit constant per block of 64, i.e. 0.5 bits per weight) the store keeps
  each block's float32 constant c itself, and w' = fl32(L4[q] * c); the
  level-1 codes are the same as with double quantization. Pinned by the
  worked example's printed values, an exact rational recomputation of
  single elements, the half-gap error bound and agreement with the
  double-quantized value wherever c' = c (a block that holds its group's
  maximum).

* Dequantization. c' = fl32(L8[q8] * s2), w' = fl32(L4[q] * c') with
  L8[k] = fl32(k / 255) ([P4] "A worked example" step 4, "Step 5: forward
  pass with on-the-fly dequantization"). Pinned by the worked example
  and the error bound |w - w'| <= c * gap/2 + |L4[q]| * |c - c'|.

Everything below uses float32 arithmetic where the stored format is float32
(as numpy float32 ops: IEEE, correctly rounded, no contraction), and exact
float64 / rational arithmetic where a decision (nearest level) is taken.
"""

import math
from fractions import Fraction
from statistics import NormalDist

import numpy as np

BLOCK = 64
GROUP = 256
# Outermost probability of the codebook, as an exact rational.
P_MAX_FRACTION = 1 - (Fraction(1, 30) + Fraction(1, 32)) / 2  # = 929/960
P_MAX = float(P_MAX_FRACTION)


# ----------------------------------------------------------------------------
# codebook
# ----------------------------------------------------------------------------

def _probabilities():
    """Probabilities whose normal quantiles become the levels.

    Positive half: 8 levels at p = 1/2 + i * (P_MAX - 1/2) / 8, i = 1..8.
    Negative half: 7 levels at p = 1/2 + i * (P_MAX - 1/2) / 7, i = 1..7,
    mirrored. Each is computed exactly as a rational and rounded once.
    """
    half = Fraction(1, 2)
    pos = [float(half + i * (P_MAX_FRACTION - half) / 8) for i in range(1, 9)]
    neg = [float(half + i * (P_MAX_FRACTION - half) / 7) for i in range(1, 8)]
    return pos, neg


def codebook_fp64(inv_cdf=None):
    """The 16 NF4 levels in float64, ascending, before rounding to float32.

    `inv_cdf` defaults to the standard library's normal quantile function;
    tests pass an independent one to pin the result.
    """
    if inv_cdf is None:
        inv_cdf = NormalDist().inv_cdf
    pos, neg = _probabilities()
    top = inv_cdf(P_MAX)
    levels = [inv_cdf(p) / top for p in pos]
    levels += [-inv_cdf(p) / top for p in neg]
    levels.append(0.0)
    return np.array(sorted(levels), dtype=np.float64)


def codebook():
    """The 16 NF4 levels as float32 (one correctly rounded conversion)."""
    return codebook_fp64().astype(np.float32)


def level8():
    """The 256 values of the 8-bit constant code: L8[k] = fl32(k / 255)."""
    return np.arange(256, dtype=np.float32) / np.float32(255.0)


# ----------------------------------------------------------------------------
# sizes
# ----------------------------------------------------------------------------

def num_blocks(numel):
    return -(-int(numel) // BLOCK)


def num_groups(numel):
    return -(-num_blocks(numel) // GROUP)


def codes_bytes(numel):
    return -(-int(numel) // 2)


def store_bytes(numel, double_quant=True):
    """Bytes of the stored tensor: packed codes + constants."""
    if double_quant:
        return codes_bytes(numel) + num_blocks(numel) + 4 * num_groups(numel)
    return codes_bytes(numel) + 4 * num_blocks(numel)


def bits_per_param(block=BLOCK, group=GROUP, double_quant=True):
    """Storage per parameter as an exact Fraction ([P4] "Step 2", "Step 3").

    Without double quantization: 4 bits + one 32-bit constant per block.
    With it: 4 bits + one 8-bit constant per block + one 32-bit constant per
    group of `group` blocks.
    """
    if double_quant:
        return 4 + Fraction(8, block) + Fraction(32, block * group)
    return 4 + Fraction(32, block)


# ----------------------------------------------------------------------------
# level 1
# ----------------------------------------------------------------------------

def nearest_level(n, levels=None):
    """Index of the nearest level to each float32 value n (ties: lower index).

    Distances are taken in float64; near any decision point n and the level
    are within a factor of two of each other's scale, so the difference of
    two float32 numbers is exact there and the decision is exact.
    """
    if levels is None:
        levels = codebook()
    n64 = np.asarray(n, dtype=np.float32).astype(np.float64)
    lv = np.asarray(levels, dtype=np.float32).astype(np.float64)
    dist = np.abs(n64[..., None] - lv)
    return np.argmin(dist, axis=-1).astype(np.uint8)  # first minimum = lower index


def _block_absmax(w):
    numel = w.size
    nb = num_blocks(numel)
    padded = np.zeros(nb * BLOCK, dtype=np.float32)
    padded[:numel] = np.abs(w)
    return padded.reshape(nb, BLOCK).max(axis=1)


def _level1_codes(w, absmax, chunk=1 << 20):
    """Unpacked codes, one uint8 per element."""
    levels = codebook()
    numel = w.size
    q = np.empty(numel, dtype=np.uint8)
    zero_code = int(nearest_level(np.float32(0.0), levels))
    for s in range(0, numel, chunk):
        e = min(numel, s + chunk)
        blk = np.arange(s, e) // BLOCK
        c = absmax[blk]
        safe = np.where(c == 0, np.float32(1.0), c).astype(np.float32)
        n = (w[s:e] / safe).astype(np.float32)  # one IEEE float32 division
        qq = nearest_level(n, levels)
        qq[c == 0] = zero_code
        q[s:e] = qq
    return q


def pack_codes(q):
    """Two 4-bit codes per byte: element 2i low nibble, 2i+1 high nibble."""
    q = np.asarray(q, dtype=np.uint8).ravel()
    if q.size % 2:
        q = np.concatenate([q, np.zeros(1, np.uint8)])
    return (q[0::2] | (q[1::2] << 4)).astype(np.uint8)


def unpack_codes(packed, numel):
    packed = np.asarray(packed, dtype=np.uint8).ravel()
    q = np.empty(packed.size * 2, dtype=np.uint8)
    q[0::2] = packed & 0x0F
    q[1::2] = packed >> 4
    return q[:numel]


# ----------------------------------------------------------------------------
# level 2
# ----------------------------------------------------------------------------

def _double_quant(absmax):
    nb = absmax.size
    ng = -(-nb // GROUP)
    padded = np.zeros(ng * GROUP, dtype=np.float32)
    padded[:nb] = absmax
    s2 = padded.reshape(ng, GROUP).max(axis=1).astype(np.float32)
    g = np.arange(nb) // GROUP
    denom = np.where(s2[g] == 0, np.float32(1.0), s2[g]).astype(np.float32)
    ratio = (absmax / denom).astype(np.float32)           # fl32(c / s2)
    scaled = (ratio * np.float32(255.0)).astype(np.float32)  # fl32(. * 255)
    q8 = np.clip(np.rint(scaled), 0, 255).astype(np.uint8)  # half-even
    q8[s2[g] == 0] = 0
    return q8, s2


# ----------------------------------------------------------------------------
# public
# ----------------------------------------------------------------------------

def quantize(w):
    """Quantize a flat float32 array (bf16-exact values) to the NF4 store.

    Returns a dict with
      codes     uint8 [ceil(numel/2)]   packed 4-bit level indices
      absmax_q  uint8 [nblocks]         8-bit codes of the block constants
      absmax_s2 float32 [ngroups]       second-level constants
      absmax    float32 [nblocks]       first-level constants (before DQ)
      q         uint8 [numel]           unpacked codes (for diagnostics)
    """
    w = np.ascontiguousarray(np.asarray(w, dtype=np.float32).ravel())
    absmax = _block_absmax(w)
    q = _level1_codes(w, absmax)
    q8, s2 = _double_quant(absmax)
    return {
        "codes": pack_codes(q),
        "absmax_q": q8,
        "absmax_s2": s2,
        "absmax": absmax,
        "q": q,
        "numel": w.size,
    }


def dequantize(codes, absmax_q, absmax_s2, numel):
    """Reconstruct float32 w' from the store (two roundings, never fused)."""
    levels = codebook()
    l8 = level8()
    q = unpack_codes(codes, numel)
    q8 = np.asarray(absmax_q, dtype=np.uint8)
    s2 = np.asarray(absmax_s2, dtype=np.float32)
    g = np.arange(q8.size) // GROUP
    cprime = (l8[q8] * s2[g]).astype(np.float32)           # fl32(L8[q8] * s2)
    blk = np.arange(numel) // BLOCK
    return (levels[q] * cprime[blk]).astype(np.float32)    # fl32(L4[q] * c')


def dequantize_nodq(codes, absmax, numel):
    """Reconstruct float32 w' from a store without double quantization:
    w' = fl32(L4[q] * c), c the float32 constant of the element's block."""
    levels = codebook()
    q = unpack_codes(codes, numel)
    c = np.asarray(absmax, dtype=np.float32)
    blk = np.arange(numel) // BLOCK
    return (levels[q] * c[blk]).astype(np.float32)
