// AdamW step for the adapter parameters, float32 state or 8-bit state.
//
// The trained parameters of the method are the adapter matrices; the pages
// name AdamW (32-bit or 8-bit state, paged) as their optimizer
// (ozercemkelahmet.com "QLoRA", "Practical guidance and best practices",
// Optimizer and schedule; same page, "How it works", Step 7: paged
// optimizers keep the state in memory that can move between device and
// host). The update is
// AdamW's: Adam's moment estimates with bias correction and a weight decay
// decoupled from the gradient. Every operation below is one float32
// operation rounded on its own (no contraction into fma; division and
// square root correctly rounded), in this order:
//   p1 = p - fl(lw * p)                       lw = fl(lr * wd)
//   m1 = fl(b1 * m) + fl(ob1 * g)             ob1 = fl(1 - b1)
//   v1 = fl(b2 * v) + fl(ob2 * fl(g * g))     ob2 = fl(1 - b2)
//   den = sqrt(fl(v1 / c2)) + eps             c2 = fl(1 - b2^t)
//   p2 = p1 - fl(lr * fl(fl(m1 / c1) / den))  c1 = fl(1 - b1^t)
// and optionally the bf16 copy of p2 (round to nearest even) that the
// linear calls take as A or B. The host constants are computed in float64
// and rounded once. The divisions by c1 and c2 (and, for the 8-bit state,
// by the block scales) are taken as float64 products with the float64
// reciprocal, rounded once to float32, which gives the correctly rounded
// quotient (div_rc below); the division by den and the square root are
// float32's own correctly rounded operations. The state may be device memory or pinned host memory
// mapped into the device's address space: the kernel streams through it in
// place either way.
#include <cmath>

#include "common.h"
#include "kernels.h"

namespace qlora {

namespace {

struct AdamWConst {
  float lr, lw, b1, ob1, b2, ob2, c1, c2, eps;
  double rc1, rc2;  // fl64(1 / c1), fl64(1 / c2)
};

// fl32(x / c) from rc = fl64(1 / c): fl32(fl64(x * rc)). Exact for every
// float32 x and positive float32 c. A quotient of two float32 values is never
// a midpoint between adjacent float32 values (a midpoint needs 25 significant
// bits, and A = M * B with A < 2^24, M >= 2^24 odd has no solution), and its
// distance from every midpoint is at least 1 / (M * B) > 2^-49 relative; the
// float64 product is within 2^-52 relative of the quotient, so it rounds to
// the same float32. Subnormal quotients only widen the margin; 0, infinities
// and NaN pass through as the division gives them.
__device__ __forceinline__ float div_rc(float x, double rc) {
  return (float)((double)x * rc);
}

__device__ __forceinline__ void adamw_one(float& p, float& m, float& v, float g,
                                          const AdamWConst& k) {
#pragma clang fp contract(off)
  const float p1 = p - k.lw * p;
  const float m1 = k.b1 * m + k.ob1 * g;
  const float v1 = k.b2 * v + k.ob2 * (g * g);
  const float den = __builtin_sqrtf(div_rc(v1, k.rc2)) + k.eps;
  p = p1 - k.lr * (div_rc(m1, k.rc1) / den);
  m = m1;
  v = v1;
}

// 16-byte accesses where the arrays allow it (n % 4 == 0 and 16-byte aligned
// pointers): two units of four parameters per thread, all eight loads issued
// before any arithmetic, non-temporal (every byte is read and written once
// per step), with a grid large enough that each thread has only its own two
// units; one parameter per thread otherwise.
template <bool kVec>
__global__ void __launch_bounds__(256)
adamw_kernel(float* __restrict__ p, float* __restrict__ m, float* __restrict__ v,
             const float* __restrict__ g, int64_t n, AdamWConst k,
             uint16_t* __restrict__ p16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  if (kVec) {
    const int64_t units = n / 4;
    for (int64_t i0 = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i0 < units; i0 += 2 * stride) {
      floatx4 pp[2], mm[2], vv[2], gg[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int64_t i = i0 + u * stride;
        if (i >= units) break;
        pp[u] = __builtin_nontemporal_load(&reinterpret_cast<floatx4*>(p)[i]);
        mm[u] = __builtin_nontemporal_load(&reinterpret_cast<floatx4*>(m)[i]);
        vv[u] = __builtin_nontemporal_load(&reinterpret_cast<floatx4*>(v)[i]);
        gg[u] = __builtin_nontemporal_load(&reinterpret_cast<const floatx4*>(g)[i]);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int64_t i = i0 + u * stride;
        if (i >= units) break;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          float a = pp[u][c], b = mm[u][c], d = vv[u][c];
          adamw_one(a, b, d, gg[u][c], k);
          pp[u][c] = a; mm[u][c] = b; vv[u][c] = d;
        }
        __builtin_nontemporal_store(pp[u], &reinterpret_cast<floatx4*>(p)[i]);
        __builtin_nontemporal_store(mm[u], &reinterpret_cast<floatx4*>(m)[i]);
        __builtin_nontemporal_store(vv[u], &reinterpret_cast<floatx4*>(v)[i]);
        if (p16) {
          const u32x2 b16 = u32x2{pack_bf16x2(pp[u][0], pp[u][1]), pack_bf16x2(pp[u][2], pp[u][3])};
          __builtin_nontemporal_store(b16, &reinterpret_cast<u32x2*>(p16)[i]);
        }
      }
    }
  } else {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += stride) {
      float a = p[i], b = m[i], d = v[i];
      adamw_one(a, b, d, g[i], k);
      p[i] = a; m[i] = b; v[i] = d;
      if (p16) p16[i] = (uint16_t)(pack_bf16x2(a, 0.0f) & 0xffffu);
    }
  }
}

// ---------------------------------------------------------------------------
// 8-bit state. Each moment is held per block of 256 parameters as 8-bit
// floating-point codes (OCP OFP8: E4M3 for m, E5M2 for v; sign, exponent
// bias 7 / 15, 3 / 2 mantissa bits, subnormals) and one float32 scale:
//   x' = fl(dec(code) * scale),   scale = fl(max_block |x| / top),
//   code = enc(fl(x / scale)) (0 when scale = 0), top = 448 / 57344,
// enc rounding to nearest, ties to the even code, saturating at top. One
// wave owns one block: four parameters per lane, the block maxima by a
// wave-wide reduction, so the new scales are uniform over the wave and
// x / scale is a product with one float64 reciprocal per wave. The
// parameter, gradient and code accesses are non-temporal: each byte is read
// and written once per step.

constexpr int kBlock8 = 256;

// gfx950's OFP8 conversions: v_cvt_f32_fp8 / v_cvt_f32_bf8 decode one byte
// exactly; v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32 encode two floats with
// rounding to nearest, ties to even, on the subnormal grid below the
// smallest normal. Inputs are first clamped to the largest finite magnitude
// (448 / 57344), which makes them saturate like the encoding above. Checked
// on gfx950 against the bit-level ofp8_encode / ofp8_decode for every
// non-NaN float32 and every non-NaN code: no difference. (A NaN, which only a
// NaN gradient brings, is not coded the same way.)
template <int kSel>
__device__ __forceinline__ float fp8_sel(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8((int)w, kSel);
}
__device__ __forceinline__ float fp8_byte(uint32_t w, int j) {
  return j == 0 ? fp8_sel<0>(w) : j == 1 ? fp8_sel<1>(w) : j == 2 ? fp8_sel<2>(w) : fp8_sel<3>(w);
}
template <int kSel>
__device__ __forceinline__ float bf8_sel(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_bf8((int)w, kSel);
}
__device__ __forceinline__ float bf8_byte(uint32_t w, int j) {
  return j == 0 ? bf8_sel<0>(w) : j == 1 ? bf8_sel<1>(w) : j == 2 ? bf8_sel<2>(w) : bf8_sel<3>(w);
}
__device__ __forceinline__ float clampf(float x, float t) { return fminf(fmaxf(x, -t), t); }
__device__ __forceinline__ uint32_t fp8_pack4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(clampf(a, 448.0f), clampf(b, 448.0f), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(clampf(c, 448.0f), clampf(d, 448.0f), lo, true);
}
__device__ __forceinline__ uint32_t bf8_pack4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_bf8_f32(clampf(a, 57344.0f), clampf(b, 57344.0f), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_bf8_f32(clampf(c, 57344.0f), clampf(d, 57344.0f), lo, true);
}

template <bool kVec>
__global__ void __launch_bounds__(256)
adamw8_kernel(float* __restrict__ p, uint8_t* __restrict__ m8, float* __restrict__ sm,
              uint8_t* __restrict__ v8, float* __restrict__ sv, const float* __restrict__ g,
              int64_t n, AdamWConst k, uint16_t* __restrict__ p16) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  const int64_t nb = (n + kBlock8 - 1) / kBlock8;
  // the block index is the same for every lane of a wave
  for (int64_t b = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); b < nb;
       b += (int64_t)gridDim.x * 4) {
    const int64_t e0 = b * kBlock8 + lane * 4;
    float pv[4], gv[4];
    uint32_t mc = 0, vc = 0;
    const bool whole = e0 + 4 <= n;
    if (kVec && whole) {
      const floatx4 a = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p + e0));
      const floatx4 c = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(g + e0));
#pragma unroll
      for (int j = 0; j < 4; ++j) { pv[j] = a[j]; gv[j] = c[j]; }
      mc = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(m8 + e0));
      vc = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(v8 + e0));
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pv[j] = 0.0f;
        gv[j] = 0.0f;
        if (e0 + j < n) {
          pv[j] = p[e0 + j];
          gv[j] = g[e0 + j];
          mc |= (uint32_t)m8[e0 + j] << (8 * j);
          vc |= (uint32_t)v8[e0 + j] << (8 * j);
        }
      }
    }
    const float smv = sm[b], svv = sv[b];
    float mv[4], vv[4];
    float am = 0.0f, av = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float m = fp8_byte(mc, j) * smv;
      float v = bf8_byte(vc, j) * svv;
      adamw_one(pv[j], m, v, gv[j], k);
      mv[j] = m;
      vv[j] = v;
      if (e0 + j < n) {
        am = fmaxf(am, fabsf(m));
        av = fmaxf(av, v);
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      am = fmaxf(am, __shfl_xor(am, off));
      av = fmaxf(av, __shfl_xor(av, off));
    }
    const float smn = am / 448.0f;      // IEEE division
    const float svn = av / 57344.0f;
    // the scales are the same for the whole wave: one float64 reciprocal each
    uint32_t mo = 0, vo = 0;
    if (smn != 0.0f) {
      const double r = 1.0 / (double)smn;
      mo = fp8_pack4(div_rc(mv[0], r), div_rc(mv[1], r), div_rc(mv[2], r), div_rc(mv[3], r));
    }
    if (svn != 0.0f) {
      const double r = 1.0 / (double)svn;
      vo = bf8_pack4(div_rc(vv[0], r), div_rc(vv[1], r), div_rc(vv[2], r), div_rc(vv[3], r));
    }
    if (kVec && whole) {
      __builtin_nontemporal_store(floatx4{pv[0], pv[1], pv[2], pv[3]}, reinterpret_cast<floatx4*>(p + e0));
      __builtin_nontemporal_store(mo, reinterpret_cast<uint32_t*>(m8 + e0));
      __builtin_nontemporal_store(vo, reinterpret_cast<uint32_t*>(v8 + e0));
      if (p16)
        __builtin_nontemporal_store(u32x2{pack_bf16x2(pv[0], pv[1]), pack_bf16x2(pv[2], pv[3])}, reinterpret_cast<u32x2*>(p16 + e0));
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (e0 + j >= n) continue;
        p[e0 + j] = pv[j];
        m8[e0 + j] = (uint8_t)(mo >> (8 * j));
        v8[e0 + j] = (uint8_t)(vo >> (8 * j));
        if (p16) p16[e0 + j] = (uint16_t)(pack_bf16x2(pv[j], 0.0f) & 0xffffu);
      }
    }
    if (lane == 0) {
      sm[b] = smn;
      sv[b] = svn;
    }
  }
}

AdamWConst adamw_const(float lr, float beta1, float beta2, float eps, float weight_decay,
                       int64_t step) {
  AdamWConst k;
  k.lr = lr;
  k.lw = (float)((double)lr * (double)weight_decay);
  k.b1 = beta1;
  k.ob1 = (float)(1.0 - (double)beta1);
  k.b2 = beta2;
  k.ob2 = (float)(1.0 - (double)beta2);
  k.c1 = (float)(1.0 - std::pow((double)beta1, (double)step));
  k.c2 = (float)(1.0 - std::pow((double)beta2, (double)step));
  k.eps = eps;
  k.rc1 = 1.0 / (double)k.c1;
  k.rc2 = 1.0 / (double)k.c2;
  return k;
}

}  // namespace

hipError_t launch_adamw8(float* p, uint8_t* m8, float* sm, uint8_t* v8, float* sv, const float* g,
                         int64_t n, float lr, float beta1, float beta2, float eps,
                         float weight_decay, int64_t step, uint16_t* p16, hipStream_t stream) {
  const AdamWConst k = adamw_const(lr, beta1, beta2, eps, weight_decay, step);
  const bool vec = ((reinterpret_cast<uintptr_t>(p) | reinterpret_cast<uintptr_t>(g)) & 15) == 0 &&
                   ((reinterpret_cast<uintptr_t>(m8) | reinterpret_cast<uintptr_t>(v8)) & 3) == 0 &&
                   (reinterpret_cast<uintptr_t>(p16) & 7) == 0;
  const int64_t nb = (n + kBlock8 - 1) / kBlock8;
  // one wave per block of 256 parameters; a capped grid strides over the rest
  int64_t blocks = (nb + 3) / 4;
  if (blocks > ((int64_t)1 << 30)) blocks = (int64_t)1 << 30;
  if (blocks < 1) blocks = 1;
  if (vec)
    hipLaunchKernelGGL(adamw8_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, p, m8, sm,
                       v8, sv, g, n, k, p16);
  else
    hipLaunchKernelGGL(adamw8_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, p, m8,
                       sm, v8, sv, g, n, k, p16);
  return hipGetLastError();
}

hipError_t launch_adamw(float* p, float* m, float* v, const float* g, int64_t n, float lr,
                        float beta1, float beta2, float eps, float weight_decay, int64_t step,
                        uint16_t* p16, hipStream_t stream) {
  const AdamWConst k = adamw_const(lr, beta1, beta2, eps, weight_decay, step);
  const bool vec = n % 4 == 0 && ((reinterpret_cast<uintptr_t>(p) | reinterpret_cast<uintptr_t>(m) |
                                   reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(g)) &
                                  15) == 0 &&
                   (reinterpret_cast<uintptr_t>(p16) & 7) == 0;
  const int64_t units = vec ? n / 4 : n;
  // two units per thread; a capped grid strides over the rest
  int64_t blocks = (units + 511) / 512;
  if (blocks > ((int64_t)1 << 30)) blocks = (int64_t)1 << 30;
  if (blocks < 1) blocks = 1;
  if (vec)
    hipLaunchKernelGGL(adamw_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, p, m, v, g,
                       n, k, p16);
  else
    hipLaunchKernelGGL(adamw_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, p, m, v,
                       g, n, k, p16);
  return hipGetLastError();
}

}  // namespace qlora
