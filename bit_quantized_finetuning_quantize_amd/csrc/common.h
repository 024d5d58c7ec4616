// Shared device-side definitions of the gfx950 NF4 library.
//
// NF4 levels: the 16 float32 values of the NormalFloat-4 type (standard
// normal quantiles at equal probability steps within each half, 7 negative,
// an exact 0 and 8 positive, scaled so the endpoints are -1 and +1;
// crackai.dev "QLoRA: Efficient Finetuning of Quantized LLMs", How It Works
// item 1; ozercemkelahmet.com "QLoRA", Why NormalFloat). The outermost
// probability is 929/960. Written as exact hexadecimal float32 literals.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

constexpr int kBlock = 64;    // values per first-level block
constexpr int kGroup = 256;   // first-level constants per second-level group

constexpr float kNF4[16] = {
    -0x1.0000000000000p+0f, -0x1.6473620000000p-1f, -0x1.0cd65c0000000p-1f,
    -0x1.94653c0000000p-2f, -0x1.2344960000000p-2f, -0x1.7a6a7a0000000p-3f,
    -0x1.74f0d20000000p-4f, 0x0.0p+0f,              0x1.45f6020000000p-4f,
    0x1.4995be0000000p-3f,  0x1.f809b40000000p-3f,  0x1.5a066c0000000p-2f,
    0x1.c3496a0000000p-2f,  0x1.200f520000000p-1f,  0x1.7227600000000p-1f,
    0x1.0000000000000p+0f,
};

// Largest float32 not above x (x is an exact double midpoint of two levels).
constexpr float round_down_f32(double x) {
  float f = static_cast<float>(x);  // nearest
  if (static_cast<double>(f) > x) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    u = (f > 0.0f) ? u - 1u : u + 1u;
    f = __builtin_bit_cast(float, u);
  }
  return f;
}


// FP4 levels (the 4-bit alternative type): the OCP MX E2M1 magnitudes
// 0, 0.5, 1, 1.5, 2, 3, 4, 6 divided by 6, so the range is [-1, 1] with an
// exact 0 and exact endpoints; sign-magnitude codes, code 8 s + m is
// (-1)^s E2M1(m) / 6 (code 8 is -0). Each division is correctly rounded, so
// each level is the float32 nearest to its exact value.
constexpr float kE2M1[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
constexpr float fp4_level(int c) { return ((c >> 3) ? -1.0f : 1.0f) * (kE2M1[c & 7] / 6.0f); }

// Store types (bit flags): the level table and the code of the block
// constants. 0 is NF4 with the 8-bit linear code.
constexpr int kStoreFP4 = 1;    // FP4 levels instead of NF4
constexpr int kStoreDqFp8 = 2;  // block constants as E4M3 codes of c / S, S = max / 448

// The levels of a store type in code order, and its constant code.
struct Codebook {
  float lv[16];
  int dq_fp8;
};
constexpr Codebook make_codebook(int store_type) {
  Codebook cb{};
  for (int c = 0; c < 16; ++c) cb.lv[c] = (store_type & kStoreFP4) ? fp4_level(c) : kNF4[c];
  cb.dq_fp8 = (store_type & kStoreDqFp8) ? 1 : 0;
  return cb;
}

// Nearest-level search for quantization: the distinct levels in ascending
// order (15 for FP4, whose +0 and -0 coincide; 16 for NF4), the decision
// thresholds between neighbours and the code of each rank. A float32 n
// takes rank #{j : n > thr[j]}. thr[j] is the largest float32 that goes to
// the lower level: below the exact midpoint, or at it when a tie goes to
// the lower level. Ties go, for NF4, to the lower code (its codes are its
// ranks: the lower level); for FP4, to the code with an even magnitude and
// then to the lower code (the E2M1 rule, and +0 over -0).
// Unused thresholds are +inf.
struct LevelSearch {
  float thr[15];
  uint8_t code[16];
  int nlev;
};
constexpr bool code_preferred(int a, int b, bool fp4) {  // a wins a tie against b
  if (fp4 && (a & 1) != (b & 1)) return (a & 1) == 0;
  return a < b;
}
constexpr float prev_f32(float f) {  // largest float32 below f (f finite, nonzero)
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u = (f > 0.0f) ? u - 1u : u + 1u;
  return __builtin_bit_cast(float, u);
}
constexpr LevelSearch make_level_search(int store_type) {
  const Codebook cb = make_codebook(store_type);
  const bool fp4 = (store_type & kStoreFP4) != 0;
  float lv[16] = {};
  int cd[16] = {};
  int n = 0;
  for (int c = 0; c < 16; ++c) {  // distinct levels, keeping the preferred code
    int k = 0;
    while (k < n && lv[k] != cb.lv[c]) ++k;
    if (k < n) {
      if (code_preferred(c, cd[k], fp4)) cd[k] = c;
    } else {
      lv[n] = cb.lv[c];
      cd[n] = c;
      ++n;
    }
  }
  for (int i = 1; i < n; ++i)  // ascending
    for (int j = i; j > 0 && lv[j - 1] > lv[j]; --j) {
      const float t = lv[j]; lv[j] = lv[j - 1]; lv[j - 1] = t;
      const int u = cd[j]; cd[j] = cd[j - 1]; cd[j - 1] = u;
    }
  LevelSearch r{};
  r.nlev = n;
  for (int j = 0; j < 15; ++j) r.thr[j] = __builtin_huge_valf();
  for (int j = 0; j + 1 < n; ++j) {
    const double mid = (static_cast<double>(lv[j]) + static_cast<double>(lv[j + 1])) * 0.5;
    const float down = round_down_f32(mid);
    const bool tie_up = !code_preferred(cd[j], cd[j + 1], fp4);
    r.thr[j] = (tie_up && static_cast<double>(down) == mid) ? prev_f32(down) : down;
  }
  for (int j = 0; j < 16; ++j) r.code[j] = (uint8_t)(j < n ? cd[j] : cd[n - 1]);
  return r;
}

// The same search by bins, one table entry per value: bin b holds the n with
// (n + 1) * 15 in [b, b + 1), b = 0 .. 31 (n below -1 clamped into bin 0,
// above 1 into the last bins). Each bin holds at most one threshold; its
// entry is that threshold (+inf if none) and the codes below and above it.
// Since no threshold lies near a bin edge (bin_search_ok), a bin index that
// the rounding of (n + 1) * 15 moves across an edge selects the same code.
constexpr int kBins = 32;
struct BinSearch {
  float thr[kBins];
  uint32_t codes[kBins];  // code below the threshold (bits 0-15), above it (bits 16-31)
};
constexpr BinSearch make_bin_search(int store_type) {
  const LevelSearch ls = make_level_search(store_type);
  BinSearch b{};
  for (int k = 0; k < kBins; ++k) {
    const double lo = k / 15.0 - 1.0, hi = (k + 1) / 15.0 - 1.0;
    int base = 0;
    float t = __builtin_huge_valf();
    for (int j = 0; j < 15; ++j) {
      const double tj = static_cast<double>(ls.thr[j]);
      if (tj < lo) ++base;
      else if (tj < hi) t = ls.thr[j];
    }
    b.thr[k] = t;
    b.codes[k] = (uint32_t)ls.code[base] | ((uint32_t)ls.code[base < 15 ? base + 1 : 15] << 16);
  }
  return b;
}
// At most one threshold per bin, and every threshold at least 1/1000 of a
// bin away from a bin edge (the rounding of (n + 1) * 15 is below 2^-19).
constexpr bool bin_search_ok(int store_type) {
  const LevelSearch ls = make_level_search(store_type);
  for (int k = 0; k < kBins; ++k) {
    const double lo = k / 15.0 - 1.0, hi = (k + 1) / 15.0 - 1.0;
    int cnt = 0;
    for (int j = 0; j < 15; ++j) {
      const double tj = static_cast<double>(ls.thr[j]);
      if (tj >= lo && tj < hi) ++cnt;
    }
    if (cnt > 1) return false;
  }
  for (int j = 0; j < 15; ++j) {
    const double tj = static_cast<double>(ls.thr[j]);
    if (tj > 1.0) continue;  // unused (+inf)
    const double x = (tj + 1.0) * 15.0;
    const double f = x - static_cast<double>(static_cast<int64_t>(x));
    if (f < 1e-3 || f > 1.0 - 1e-3) return false;
  }
  return true;
}
static_assert(bin_search_ok(0), "NF4 thresholds fit the bins");
static_assert(bin_search_ok(kStoreFP4), "FP4 thresholds fit the bins");

// NF4: 16 distinct levels whose codes are their ranks, each threshold the
// largest float32 not above the exact midpoint (ties to the lower level).
constexpr bool nf4_search_is_plain() {
  const LevelSearch ls = make_level_search(0);
  if (ls.nlev != 16) return false;
  for (int j = 0; j < 16; ++j)
    if (ls.code[j] != j) return false;
  for (int j = 0; j < 15; ++j)
    if (ls.thr[j] != round_down_f32((static_cast<double>(kNF4[j]) + kNF4[j + 1]) * 0.5))
      return false;
  return true;
}
static_assert(nf4_search_is_plain(), "NF4 level search");
static_assert(make_level_search(kStoreFP4).nlev == 15, "FP4 has 15 distinct levels");

// ---------------------------------------------------------------------------
// vector types
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// float32 -> bfloat16 bits, round to nearest even (v_cvt_pk_bf16_f32).
// Two floats -> bf16x2 (RNE), lo in bits 0..15: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// Level lookups for the 8 codes of one dword (element 2j in the low nibble
// of byte j). Byte j of lo4 is 4 x the low nibble, a byte offset into `lv`
// (the 16 levels, 4-byte stride); byte j of hi16 is 16 x the high nibble, a
// byte offset into `lv16` (the levels at a 16-byte stride). Each lookup
// address is then one byte extract. The masks are formed in asm so that the
// compiler cannot fold them back into a shift and a mask per element.
struct CodeOffsets {
  uint32_t lo4, hi16;
};
__device__ __forceinline__ CodeOffsets code_offsets(uint32_t word) {
  CodeOffsets o;
  asm("v_lshlrev_b32 %0, 2, %1\n\tv_and_b32 %0, 0x3c3c3c3c, %0" : "=&v"(o.lo4) : "v"(word));
  asm("v_and_b32 %0, 0xf0f0f0f0, %1" : "=v"(o.hi16) : "v"(word));
  return o;
}
__device__ __forceinline__ float level_lo(const float* lv, CodeOffsets o, int j) {
  return *reinterpret_cast<const float*>(reinterpret_cast<const char*>(lv) +
                                         ((o.lo4 >> (8 * j)) & 0xffu));
}
__device__ __forceinline__ float level_hi(const float* lv16, CodeOffsets o, int j) {
  return *reinterpret_cast<const float*>(reinterpret_cast<const char*>(lv16) +
                                         ((o.hi16 >> (8 * j)) & 0xffu));
}

// Lookups without LDS, for one block constant cs and the 16 levels lv of
// the store type (in code order). The 16 possible weights
// bf16(fl32(L[q] * cs)) are computed once (16 multiplies, the same two
// roundings as every other path) and split into a low-byte plane and a
// high-byte plane of 16 bytes each (4 dwords, entry q in byte q % 4 of dword
// q / 4). A code then selects its two bytes with v_perm_b32: one perm over
// entries 0-7, one over entries 8-15, and a byte mask from bit 3 of the code
// picks between them.
struct PermTable {
  uint32_t lo[4], hi[4];
};
__device__ __forceinline__ PermTable perm_table(float cs, const float (&lv)[16]) {
#pragma clang fp contract(off)
  uint32_t pk[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) pk[i] = pack_bf16x2(lv[2 * i] * cs, lv[2 * i + 1] * cs);
  PermTable t;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    t.lo[k] = __builtin_amdgcn_perm(pk[2 * k + 1], pk[2 * k], 0x06040200u);
    t.hi[k] = __builtin_amdgcn_perm(pk[2 * k + 1], pk[2 * k], 0x07050301u);
  }
  return t;
}
// sel: four codes, one per byte, in bits 0-2 of the byte; mask: 0xff in the
// bytes whose code is >= 8. Returns the four selected bytes of plane p.
__device__ __forceinline__ uint32_t perm_lookup(const uint32_t (&p)[4], uint32_t sel,
                                                uint32_t mask) {
  const uint32_t a = __builtin_amdgcn_perm(p[1], p[0], sel);
  const uint32_t b = __builtin_amdgcn_perm(p[3], p[2], sel);
  return (b & mask) | (a & ~mask);
}
// 8 codes -> 4 words of bf16 pairs bf16(fl32(L[q] * cs)) (the two roundings
// happen once per table entry, in perm_table).
__device__ __forceinline__ u32x4 dequant_word_perm(uint32_t w, const PermTable& t) {
  // byte masks from bit 3 of each code: v_perm selector 8 (9, 10, 11) copies
  // bit 7 of byte 1 (3, 5, 7) of its source pair into a whole byte
  const uint32_t m_lo = __builtin_amdgcn_perm(w << 4, w << 12, 0x0B090A08u);
  const uint32_t m_hi = __builtin_amdgcn_perm(w, w << 8, 0x0B090A08u);
  const uint32_t s_lo = w & 0x07070707u, s_hi = (w >> 4) & 0x07070707u;
  const uint32_t x = perm_lookup(t.lo, s_lo, m_lo);  // low bytes, even elements
  const uint32_t y = perm_lookup(t.hi, s_lo, m_lo);  // high bytes, even elements
  const uint32_t z = perm_lookup(t.lo, s_hi, m_hi);  // low bytes, odd elements
  const uint32_t v = perm_lookup(t.hi, s_hi, m_hi);  // high bytes, odd elements
  const uint32_t xy01 = __builtin_amdgcn_perm(y, x, 0x05010400u);
  const uint32_t xy23 = __builtin_amdgcn_perm(y, x, 0x07030602u);
  const uint32_t zv01 = __builtin_amdgcn_perm(v, z, 0x05010400u);
  const uint32_t zv23 = __builtin_amdgcn_perm(v, z, 0x07030602u);
  return u32x4{__builtin_amdgcn_perm(zv01, xy01, 0x05040100u),
               __builtin_amdgcn_perm(zv01, xy01, 0x07060302u),
               __builtin_amdgcn_perm(zv23, xy23, 0x05040100u),
               __builtin_amdgcn_perm(zv23, xy23, 0x07060302u)};
}

// The same lookups with the elements left in the order 0, 2, 4, 6, 1, 3, 5, 7
// (word 0 holds elements 0 and 2, word 1 elements 4 and 6, word 2 elements
// 1 and 3, word 3 elements 5 and 7): one byte interleave per output word
// instead of two. A contraction that takes its other operand in the same
// order (x_order_oddeven) sums the same products.
__device__ __forceinline__ u32x4 dequant_word_perm_oddeven(uint32_t w, const PermTable& t) {
  const uint32_t m_lo = __builtin_amdgcn_perm(w << 4, w << 12, 0x0B090A08u);
  const uint32_t m_hi = __builtin_amdgcn_perm(w, w << 8, 0x0B090A08u);
  const uint32_t s_lo = w & 0x07070707u, s_hi = (w >> 4) & 0x07070707u;
  const uint32_t xl = perm_lookup(t.lo, s_lo, m_lo);  // low bytes, even elements
  const uint32_t xh = perm_lookup(t.hi, s_lo, m_lo);  // high bytes, even elements
  const uint32_t zl = perm_lookup(t.lo, s_hi, m_hi);  // low bytes, odd elements
  const uint32_t zh = perm_lookup(t.hi, s_hi, m_hi);  // high bytes, odd elements
  return u32x4{__builtin_amdgcn_perm(xh, xl, 0x05010400u), __builtin_amdgcn_perm(xh, xl, 0x07030602u),
               __builtin_amdgcn_perm(zh, zl, 0x05010400u), __builtin_amdgcn_perm(zh, zl, 0x07030602u)};
}
// Eight consecutive bf16 values (word j holds elements 2j, 2j + 1) put in
// the element order of dequant_word_perm_oddeven.
__device__ __forceinline__ u32x4 x_order_oddeven(const u32x4& v) {
  return u32x4{__builtin_amdgcn_perm(v[1], v[0], 0x05040100u), __builtin_amdgcn_perm(v[3], v[2], 0x05040100u),
               __builtin_amdgcn_perm(v[1], v[0], 0x07060302u), __builtin_amdgcn_perm(v[3], v[2], 0x07060302u)};
}

__device__ __forceinline__ float bf16_lo(uint32_t v) {
  return __builtin_bit_cast(float, v << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t v) {
  return __builtin_bit_cast(float, v & 0xffff0000u);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t v) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(v) << 16);
}

// OCP 8-bit floating-point codes (OFP8; sign, kE exponent bits with bias
// kBias, kM mantissa bits, subnormals). dec: the value of a code, exactly
// (the exponent field goes straight into the float's exponent; subnormals
// are m 2^(1 - bias - kM)).
template <int kE, int kM, int kBias>
__device__ __forceinline__ float ofp8_decode(uint32_t c) {
  const uint32_t s = (c >> 7) & 1u;
  const uint32_t e = (c >> kM) & ((1u << kE) - 1u);
  const uint32_t m = c & ((1u << kM) - 1u);
  const float sub = (float)m * __builtin_bit_cast(float, (uint32_t)(127 + 1 - kBias - kM) << 23);
  const float nrm = __builtin_bit_cast(float, ((e + 127u - kBias) << 23) | (m << (23 - kM)));
  const float mag = e ? nrm : sub;
  return s ? -mag : mag;
}

// enc for a finite float: the mantissa rounded to kM bits on its integer
// bits (ties to even), a carry running into the exponent field; values
// below the smallest normal rounded on the subnormal grid; saturating at
// kTopCode.
template <int kE, int kM, int kBias, uint32_t kTopCode>
__device__ __forceinline__ uint32_t ofp8_encode(float y) {
  const uint32_t u = __builtin_bit_cast(uint32_t, y);
  const uint32_t sign = (u >> 31) << 7;
  const uint32_t ua = u & 0x7fffffffu;
  const float a = __builtin_bit_cast(float, ua);
  const float top = ofp8_decode<kE, kM, kBias>(kTopCode);
  const float min_normal = __builtin_bit_cast(float, (uint32_t)(127 + 1 - kBias) << 23);
  uint32_t mag;
  if (!(a < top)) {
    mag = kTopCode;
  } else if (a < min_normal) {
    // a 2^(bias - 1 + kM) is exact; rintf rounds half to even
    mag = (uint32_t)__builtin_rintf(a * __builtin_bit_cast(float, (uint32_t)(127 - 1 + kBias + kM) << 23));
  } else {
    const uint32_t e = (ua >> 23) - 127u + kBias;     // biased exponent of the code
    const uint32_t q = (ua >> (23 - kM)) & ((1u << kM) - 1u);
    const uint32_t rem = ua & ((1u << (23 - kM)) - 1u);
    const uint32_t half = 1u << (22 - kM);
    const uint32_t up = (rem > half || (rem == half && (q & 1u))) ? 1u : 0u;
    mag = ((e << kM) + q + up);
    mag = mag > kTopCode ? kTopCode : mag;
  }
  return mag | sign;
}
__device__ __forceinline__ float e4m3_decode(uint32_t c) { return ofp8_decode<4, 3, 7>(c); }

// Second-level dequantization of a block constant:
//   c' = fl32( fl32(q8 / 255) * s2 )   (two separately rounded operations)
__device__ __forceinline__ float block_scale(uint32_t q8, float s2) {
#pragma clang fp contract(off)
  const float l8 = static_cast<float>(q8) / 255.0f;  // IEEE division
  return l8 * s2;
}
// ... and with the 8-bit floating-point code: c' = fl32(dec(q8) * S)
// (dec exact), S the group's scale.
__device__ __forceinline__ float block_scale_fp8(uint32_t q8, float S) {
#pragma clang fp contract(off)
  return e4m3_decode(q8) * S;
}
// The value of 8-bit constant code k of a store (for the LDS table that the
// MFMA loaders read): fl32(k / 255), or the E4M3 value.
__device__ __forceinline__ float level8_of(int k, int dq_fp8) {
#pragma clang fp contract(off)
  return dq_fp8 ? e4m3_decode((uint32_t)k) : static_cast<float>(k) / 255.0f;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

}  // namespace qlora
