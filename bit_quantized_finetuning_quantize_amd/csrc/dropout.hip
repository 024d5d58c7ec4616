// Keep mask of LoRA dropout on the adapter input.
//
// ozercemkelahmet.com "QLoRA": the LoraConfig of "A code example with common
// libraries" trains with a LoRA dropout of 0.05, and "Practical guidance and
// best practices", Adapter settings, recommends a small dropout rate when
// the training data is scarce. Each element of the [M x K] adapter input is
// kept independently with probability 1 - thr / 2^16.
//
// Random numbers: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
// random numbers: as easy as 1, 2, 3", SC'11): key = the 64-bit seed, counter
// = (g, offset) for group g of eight consecutive elements in row-major order;
// output word w gives elements 8g + 2w (low half) and 8g + 2w + 1 (high
// half). Counter-based, so any kernel can regenerate any element's draw, and
// a mask can be rebuilt from (seed, offset) instead of being kept.
//
// One thread per mask word: 32 elements = four generator calls; consecutive
// threads write consecutive words.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace qlora {

namespace {

__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    c = u32x4{(uint32_t)(p1 >> 32) ^ c[1] ^ k0, (uint32_t)p1, (uint32_t)(p0 >> 32) ^ c[3] ^ k1,
              (uint32_t)p0};
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

__global__ void __launch_bounds__(256)
dropout_mask_kernel(uint32_t* __restrict__ mask, int64_t words, uint32_t thr, uint32_t k0,
                    uint32_t k1, uint32_t o0, uint32_t o1) {
  for (int64_t wi = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; wi < words;
       wi += (int64_t)gridDim.x * blockDim.x) {
    uint32_t bits = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint64_t g = (uint64_t)wi * 4 + c;
      const u32x4 x = philox4x32_10(u32x4{(uint32_t)g, (uint32_t)(g >> 32), o0, o1}, k0, k1);
#pragma unroll
      for (int h = 0; h < 8; ++h) {
        const uint32_t v = (x[h >> 1] >> (16 * (h & 1))) & 0xffffu;
        bits |= (uint32_t)(v >= thr) << (8 * c + h);
      }
    }
    mask[wi] = bits;
  }
}

}  // namespace

hipError_t launch_dropout_mask(int64_t M, int64_t K, uint32_t thr, uint64_t seed,
                               uint64_t offset, uint32_t* mask, hipStream_t stream) {
  const int64_t words = M * (K / 32);
  const int64_t blocks = std::min<int64_t>((words + 255) / 256, 16384);
  hipLaunchKernelGGL(dropout_mask_kernel, dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(256),
                     0, stream, mask, words, thr, (uint32_t)seed, (uint32_t)(seed >> 32),
                     (uint32_t)offset, (uint32_t)(offset >> 32));
  return hipGetLastError();
}

}  // namespace qlora
