// AdamW step for the adapter parameters, float32 state.
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
// and rounded once. The state may live in any memory the device can access
// (device, or managed memory that pages to the host): the kernel only
// streams through it.
#include <cmath>

#include "common.h"
#include "kernels.h"

namespace qlora {

namespace {

struct AdamWConst {
  float lr, lw, b1, ob1, b2, ob2, c1, c2, eps;
};

__device__ __forceinline__ void adamw_one(float& p, float& m, float& v, float g,
                                          const AdamWConst& k) {
#pragma clang fp contract(off)
  const float p1 = p - k.lw * p;
  const float m1 = k.b1 * m + k.ob1 * g;
  const float v1 = k.b2 * v + k.ob2 * (g * g);
  const float den = __builtin_sqrtf(v1 / k.c2) + k.eps;
  p = p1 - k.lr * ((m1 / k.c1) / den);
  m = m1;
  v = v1;
}

// Four parameters per thread and 16-byte accesses where the arrays allow it
// (n % 4 == 0 and 16-byte aligned pointers); one parameter per thread
// otherwise.
template <bool kVec>
__global__ void __launch_bounds__(256)
adamw_kernel(float* __restrict__ p, float* __restrict__ m, float* __restrict__ v,
             const float* __restrict__ g, int64_t n, AdamWConst k,
             uint16_t* __restrict__ p16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  if (kVec) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n / 4; i += stride) {
      floatx4 pp = reinterpret_cast<floatx4*>(p)[i];
      floatx4 mm = reinterpret_cast<floatx4*>(m)[i];
      floatx4 vv = reinterpret_cast<floatx4*>(v)[i];
      const floatx4 gg = reinterpret_cast<const floatx4*>(g)[i];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float a = pp[c], b = mm[c], d = vv[c];
        adamw_one(a, b, d, gg[c], k);
        pp[c] = a; mm[c] = b; vv[c] = d;
      }
      reinterpret_cast<floatx4*>(p)[i] = pp;
      reinterpret_cast<floatx4*>(m)[i] = mm;
      reinterpret_cast<floatx4*>(v)[i] = vv;
      if (p16)
        reinterpret_cast<u32x2*>(p16)[i] = u32x2{pack_bf16x2(pp[0], pp[1]), pack_bf16x2(pp[2], pp[3])};
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

}  // namespace

hipError_t launch_adamw(float* p, float* m, float* v, const float* g, int64_t n, float lr,
                        float beta1, float beta2, float eps, float weight_decay, int64_t step,
                        uint16_t* p16, hipStream_t stream) {
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
  const bool vec = n % 4 == 0 && ((reinterpret_cast<uintptr_t>(p) | reinterpret_cast<uintptr_t>(m) |
                                   reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(g)) &
                                  15) == 0 &&
                   (reinterpret_cast<uintptr_t>(p16) & 7) == 0;
  const int64_t units = vec ? n / 4 : n;
  int64_t blocks = (units + 255) / 256;
  if (blocks > 8192) blocks = 8192;
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
