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

// Decision thresholds: for a float32 n, "n > kThr[j]" holds exactly when n
// is strictly closer to level j+1 than to level j, because kThr[j] is the
// largest float32 not above the exact midpoint. Counting the thresholds that
// n exceeds therefore gives the nearest level with ties to the lower index.
struct Thresholds {
  float t[15];
};
constexpr Thresholds make_thresholds() {
  Thresholds r{};
  for (int j = 0; j < 15; ++j)
    r.t[j] = round_down_f32((static_cast<double>(kNF4[j]) +
                             static_cast<double>(kNF4[j + 1])) * 0.5);
  return r;
}
constexpr Thresholds kThr = make_thresholds();

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

// NF4 level q from immediates (a select chain), without a memory load.
__device__ __forceinline__ float nf4_level(int q) {
  float v = kNF4[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) v = (q == i) ? kNF4[i] : v;
  return v;
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

// The 32 levels of a 16-byte packet of codes, all lookups issued before any
// use so that one LDS round trip covers them (the empty asm with a memory
// clobber keeps the compiler from interleaving each lookup with its use).
// lo[4 w + j] / hi[4 w + j]: the low / high nibble of byte j of word w.
__device__ __forceinline__ void packet_levels(const u32x4& c, const float* lv, const float* lv16,
                                              float (&lo)[16], float (&hi)[16]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const CodeOffsets o = code_offsets(c[w]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo[4 * w + j] = level_lo(lv, o, j);
      hi[4 * w + j] = level_hi(lv16, o, j);
    }
  }
  asm volatile("" ::: "memory");
}

// Lookups without LDS, for one block constant cs. The 16 possible weights
// bf16(fl32(L[q] * cs)) are computed once (16 multiplies, the same two
// roundings as every other path) and split into a low-byte plane and a
// high-byte plane of 16 bytes each (4 dwords, entry q in byte q % 4 of dword
// q / 4). A code then selects its two bytes with v_perm_b32: one perm over
// entries 0-7, one over entries 8-15, and a byte mask from bit 3 of the code
// picks between them.
struct PermTable {
  uint32_t lo[4], hi[4];
};
__device__ __forceinline__ PermTable perm_table(float cs) {
#pragma clang fp contract(off)
  uint32_t pk[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) pk[i] = pack_bf16x2(kNF4[2 * i] * cs, kNF4[2 * i + 1] * cs);
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
// 8 codes -> 4 words of bf16 pairs, bit-identical to dequant_word8.
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

// 8 codes -> 4 words of bf16 pairs bf16(fl32(L[q] * cs)): two roundings,
// never fused.
__device__ __forceinline__ u32x4 dequant_word8(uint32_t word, float cs, const float* lv,
                                               const float* lv16) {
#pragma clang fp contract(off)
  const CodeOffsets o = code_offsets(word);
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = pack_bf16x2(level_lo(lv, o, j) * cs, level_hi(lv16, o, j) * cs);
  return r;
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

// Second-level dequantization of a block constant:
//   c' = fl32( fl32(q8 / 255) * s2 )   (two separately rounded operations)
__device__ __forceinline__ float block_scale(uint32_t q8, float s2) {
#pragma clang fp contract(off)
  const float l8 = static_cast<float>(q8) / 255.0f;  // IEEE division
  return l8 * s2;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

}  // namespace qlora
