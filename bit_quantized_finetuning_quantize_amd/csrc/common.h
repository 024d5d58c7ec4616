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
