// NF4 quantization (with double quantization) and dequantization kernels.
// A null absmax_q selects the store without double quantization (Step 2
// alone): absmax_s2 then holds one float32 constant per block, c' = c.
//
// Quantization follows ozercemkelahmet.com "QLoRA", How it works, Step 1
// (blocks of 64 scaled by their largest magnitude, each value replaced by
// the nearest of 16 NormalFloat levels), Step 2 (one constant per block) and
// Step 3 (block maxima stored as 8-bit fractions of one float32 maximum per
// group of 256 blocks); ai360xpert.com "QLoRA", How It Works item 2 (the
// per-block constants shrink from 32 to 8 bits).
//
// Layout of one launch: one workgroup of 512 lanes per group of 256 blocks
// (16384 values). Within a workgroup, eight consecutive lanes own one block
// (8 values each, one 16-byte load), so every load instruction of a wave
// reads 1 KiB of contiguous HBM and a block maximum is three DPP steps. A
// workgroup loads its group in 4 rounds of 64 blocks, all loads issued before
// the first reduction, and keeps the values in registers, so each input byte
// is read once. The nearest level is found without a search: n maps to one
// of 32 bins of width 1/15 on [-1, 1], and each bin holds at most one
// threshold between levels, so one table read and one comparison give the
// code.
#include "common.h"
#include "kernels.h"

namespace qlora {

namespace {

#ifndef QUANT_THREADS
#define QUANT_THREADS 512
#endif
constexpr int kQuantThreads = QUANT_THREADS;
constexpr int kRounds = kGroup * kBlock / (kQuantThreads * 8);
static_assert(kQuantThreads >= kGroup && kRounds >= 1, "one thread per block constant");

// The code of the nearest level of n: one entry of the bin table (LDS,
// 8 bytes per bin: the bin's threshold and the codes below and above it;
// NF4 keeps only the code below, as the code above is the next one).
// NaN, which every threshold comparison leaves at rank 0, lands in bin 0 by
// the clamp (maxNum), where n > thr is false: the code of rank 0, as the
// threshold count gives it. Values beyond +-1 clamp into the outer bins.
template <bool kFP4>
__device__ __forceinline__ uint32_t bin_code(float n, const u32x2* bins) {
  const float x = fminf(fmaxf(__builtin_fmaf(n, 15.0f, 15.0f), 0.0f), (float)(kBins - 1));
  const u32x2 e = bins[(int)x];
  const bool above = n > __builtin_bit_cast(float, e.x);
  if constexpr (kFP4) return (e.y >> (above ? 16u : 0u)) & 0xfu;
  return e.y + (above ? 1u : 0u);
}

// A lane's value from another lane of its row, by a DPP control word.
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}

// kFP4: FP4 levels (sign-magnitude codes); else NF4 (the code is the rank).
// dq_fp8: the block constants as E4M3 codes of c / S with S = fl(max / 448)
// per group (else the linear code).
template <bool kVec, bool kFP4>
__global__ void __launch_bounds__(kQuantThreads)
nf4_quantize_kernel(const uint16_t* __restrict__ w, int64_t numel,
                    uint8_t* __restrict__ codes, uint8_t* __restrict__ absmax_q,
                    float* __restrict__ absmax_s2, int dq_fp8) {
#pragma clang fp contract(off)
  constexpr BinSearch kBS = make_bin_search(kFP4 ? kStoreFP4 : 0);
  constexpr uint32_t kZeroCode = kFP4 ? 0u : 7u;  // the code of level 0
  __shared__ float s_blockmax[kGroup];
  __shared__ float s_wavemax[kQuantThreads / 64];
  __shared__ u32x2 s_bins[kBins];

  const int tid = threadIdx.x;
  if (tid < kBins)  // visible after the first barrier
    s_bins[tid] = u32x2{__builtin_bit_cast(uint32_t, kBS.thr[tid]),
                        kFP4 ? kBS.codes[tid] : (kBS.codes[tid] & 0xFFFFu)};
  const int64_t nbytes = (numel + 1) / 2;
  const int64_t nblocks = (numel + kBlock - 1) / kBlock;
  const int64_t group = blockIdx.x;
  const int64_t gbase = group * (int64_t)(kGroup * kBlock);

  uint32_t vals[kRounds][4];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int64_t e0 = gbase + (int64_t)r * (kQuantThreads * 8) + tid * 8;
    if (kVec && e0 + 8 <= numel) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(w + e0);
      vals[r][0] = v.x; vals[r][1] = v.y; vals[r][2] = v.z; vals[r][3] = v.w;
    } else {
      uint16_t h[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = (e0 + i < numel) ? w[e0 + i] : (uint16_t)0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vals[r][i] = (uint32_t)h[2 * i] | ((uint32_t)h[2 * i + 1] << 16);
    }
  }

  float cmax[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m = fmaxf(m, fabsf(bf16_lo(vals[r][i])));
      m = fmaxf(m, fabsf(bf16_hi(vals[r][i])));
    }
    // the 8 lanes of a block are consecutive and aligned to 8 inside a
    // wave: swap neighbours, then pairs (quad permutations), then mirror
    // each half-row of 8 lanes, which pairs the two quads of a block
    m = fmaxf(m, dpp_f32<0xB1>(m));   // quad_perm [1,0,3,2]
    m = fmaxf(m, dpp_f32<0x4E>(m));   // quad_perm [2,3,0,1]
    m = fmaxf(m, dpp_f32<0x141>(m));  // row_half_mirror
    cmax[r] = m;
    if ((tid & 7) == 0) s_blockmax[r * (kQuantThreads / 8) + tid / 8] = m;
  }
  __syncthreads();

  // second level: group maximum over the 256 block constants
  float gm = tid < kGroup ? s_blockmax[tid] : 0.0f;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) gm = fmaxf(gm, __shfl_xor(gm, off));
  if ((tid & 63) == 0) s_wavemax[tid / 64] = gm;
  __syncthreads();
  float s2 = s_wavemax[0];
#pragma unroll
  for (int i = 1; i < kQuantThreads / 64; ++i) s2 = fmaxf(s2, s_wavemax[i]);

  const int64_t b = group * kGroup + tid;
  if (absmax_q && dq_fp8) {
    // 8-bit floating-point constant code: S = fl(max / 448), q8 = E4M3 of
    // fl(c / S) (nearest, ties to even, saturating at 448)
    const float S = s2 / 448.0f;  // IEEE division
    if (tid < kGroup && b < nblocks) {
      const uint32_t q8 = S > 0.0f ? ofp8_encode<4, 3, 7, 0x7Eu>(s_blockmax[tid] / S) : 0u;
      absmax_q[b] = (uint8_t)q8;
    }
    if (tid == 0) absmax_s2[group] = S;
  } else if (absmax_q) {
    if (tid < kGroup && b < nblocks) {
      uint32_t q8 = 0;
      if (s2 > 0.0f) {
        const float ratio = s_blockmax[tid] / s2;   // IEEE division
        const float scaled = ratio * 255.0f;
        q8 = (uint32_t)fminf(fmaxf(rintf(scaled), 0.0f), 255.0f);  // half-even
      }
      absmax_q[b] = (uint8_t)q8;
    }
    if (tid == 0) absmax_s2[group] = s2;
  } else {
    // no double quantization: the float32 block constants themselves
    if (tid < kGroup && b < nblocks) absmax_s2[b] = s_blockmax[tid];
  }

  // first level: codes against the exact float32 block maximum
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int64_t e0 = gbase + (int64_t)r * (kQuantThreads * 8) + tid * 8;
    if (e0 >= numel) continue;
    const float c = cmax[r];
    // n = w / c. For c in [2^-100, 2^100] the product with v_rcp_f32(c) gives
    // the same NF4 index as the correctly rounded quotient for every bf16
    // pair |w| <= c (checked exhaustively on gfx950: 1,065,402,238 pairs, no
    // difference inside that range, differences only beyond it, where the
    // reciprocal leaves the normal range); outside it the IEEE division.
    // (the reciprocal was checked against the NF4 thresholds only: FP4
    // divides)
    float n[8];
    if (!kFP4 && c >= 0x1p-100f && c <= 0x1p100f) {
      const float rc = __builtin_amdgcn_rcpf(c);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        n[2 * i] = bf16_lo(vals[r][i]) * rc;
        n[2 * i + 1] = bf16_hi(vals[r][i]) * rc;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        n[2 * i] = bf16_lo(vals[r][i]) / c;   // IEEE division
        n[2 * i + 1] = bf16_hi(vals[r][i]) / c;
      }
    }
    // every lane looks up all 8 codes (all table reads in flight
    // together); a block whose constant is not positive (all zeros) takes
    // the code of level 0 throughout, and nibbles past the end of the
    // tensor stay 0
    uint32_t q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = bin_code<kFP4>(n[i], s_bins);
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) word |= q[i] << (4 * i);
    if (!(c > 0.0f)) word = kZeroCode * 0x11111111u;
    const int64_t rem = numel - e0;
    if (rem < 8) word &= (1u << (4 * (int)rem)) - 1u;
    const int64_t byte0 = e0 / 2;
    if (byte0 + 4 <= nbytes) {
      // streamed out: nothing reads the codes back in this launch
      __builtin_nontemporal_store(word, reinterpret_cast<uint32_t*>(codes + byte0));
    } else {
      for (int i = 0; i < 4; ++i)
        if (byte0 + i < nbytes) codes[byte0 + i] = (uint8_t)(word >> (8 * i));
    }
  }
}

// Dequantization: 8 values per 32-bit code word, two words per thread (a
// stride of the grid apart, so that both loads are in flight together:
// 10-15 % faster than one word per thread).
template <bool kBf16>
__global__ void __launch_bounds__(256)
nf4_dequantize_kernel(const uint8_t* __restrict__ codes,
                      const uint8_t* __restrict__ absmax_q,
                      const float* __restrict__ absmax_s2, int64_t numel,
                      void* __restrict__ out, Codebook cb) {
#pragma clang fp contract(off)
  __shared__ float s_lv[16];
  if (threadIdx.x < 16) s_lv[threadIdx.x] = cb.lv[threadIdx.x];
  __syncthreads();
  const int64_t nwords = (numel + 7) / 8;
  const int64_t nbytes = (numel + 1) / 2;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i0 = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i0 < nwords; i0 += 2 * stride)
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int64_t i = i0 + u * stride;
    if (i >= nwords) break;
    const int64_t e0 = i * 8;
    uint32_t word;
    if (i * 4 + 4 <= nbytes) {
      word = *reinterpret_cast<const uint32_t*>(codes + i * 4);
    } else {
      word = 0;
      for (int j = 0; j < 4; ++j)
        if (i * 4 + j < nbytes) word |= (uint32_t)codes[i * 4 + j] << (8 * j);
    }
    const int64_t b = e0 / kBlock;
    const float cs = !absmax_q ? absmax_s2[b]
                     : cb.dq_fp8 ? block_scale_fp8(absmax_q[b], absmax_s2[b / kGroup])
                                 : block_scale(absmax_q[b], absmax_s2[b / kGroup]);
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = s_lv[(word >> (4 * j)) & 15u] * cs;
    if (kBf16) {
      uint16_t* o = reinterpret_cast<uint16_t*>(out);
      if (e0 + 8 <= numel) {
        u32x4 p;
        p.x = pack_bf16x2(v[0], v[1]);
        p.y = pack_bf16x2(v[2], v[3]);
        p.z = pack_bf16x2(v[4], v[5]);
        p.w = pack_bf16x2(v[6], v[7]);
        *reinterpret_cast<u32x4*>(o + e0) = p;
      } else {
        for (int j = 0; j < 8; ++j)
          if (e0 + j < numel)
            o[e0 + j] = (uint16_t)(pack_bf16x2(v[j], 0.0f) & 0xffffu);
      }
    } else {
      float* o = reinterpret_cast<float*>(out);
      if (e0 + 8 <= numel) {
        floatx4 a = {v[0], v[1], v[2], v[3]};
        floatx4 c = {v[4], v[5], v[6], v[7]};
        *reinterpret_cast<floatx4*>(o + e0) = a;
        *reinterpret_cast<floatx4*>(o + e0 + 4) = c;
      } else {
        for (int j = 0; j < 8; ++j)
          if (e0 + j < numel) o[e0 + j] = v[j];
      }
    }
  }
}

}  // namespace

hipError_t launch_nf4_quantize(const uint16_t* w, int64_t numel, uint8_t* codes,
                               uint8_t* absmax_q, float* absmax_s2, int store_type,
                               hipStream_t stream) {
  const int64_t ngroups = (numel + (int64_t)kGroup * kBlock - 1) / ((int64_t)kGroup * kBlock);
  const bool vec = (reinterpret_cast<uintptr_t>(w) % 16) == 0;
  const bool fp4 = (store_type & kStoreFP4) != 0;
  const int dq_fp8 = (store_type & kStoreDqFp8) ? 1 : 0;
  dim3 grid((unsigned)ngroups), block(kQuantThreads);
  if (vec && !fp4)
    hipLaunchKernelGGL((nf4_quantize_kernel<true, false>), grid, block, 0, stream, w, numel,
                       codes, absmax_q, absmax_s2, dq_fp8);
  else if (!fp4)
    hipLaunchKernelGGL((nf4_quantize_kernel<false, false>), grid, block, 0, stream, w, numel,
                       codes, absmax_q, absmax_s2, dq_fp8);
  else if (vec)
    hipLaunchKernelGGL((nf4_quantize_kernel<true, true>), grid, block, 0, stream, w, numel,
                       codes, absmax_q, absmax_s2, dq_fp8);
  else
    hipLaunchKernelGGL((nf4_quantize_kernel<false, true>), grid, block, 0, stream, w, numel,
                       codes, absmax_q, absmax_s2, dq_fp8);
  return hipGetLastError();
}

// Adapter merge (ozercemkelahmet.com "QLoRA", How it works, Step 8: save
// and use, the option that dequantizes the base to 16 bits and merges the
// adapter; same page, "Merging after QLoRA"):
//   out[n][k] = bf16( w'[n][k] + s * sum_j A[k][j] B[j][n] )
// with the sum in float32 from j = 0 upward (each product of two bf16
// values is exact, so one fma per term rounds exactly like an add), then
// fl32(s * sum), fl32(w' + that) and one round-to-nearest-even to bf16.
// Workgroup: 64 weight rows x 64 columns (one block per row); thread: two
// rows x eight columns (one code dword per row). The adapter is staged in
// LDS as float32 in chunks of 32 ranks: A transposed ([j][k]) and B as is
// ([j][n]).
constexpr int kMergeRC = 32;
__global__ void __launch_bounds__(256)
nf4_merge_kernel(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ absmax_q,
                 const float* __restrict__ absmax_s2, int64_t N, int64_t K,
                 const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, int r,
                 float s, uint16_t* __restrict__ out, Codebook cb) {
#pragma clang fp contract(off)
  __shared__ float s_lv[16];
  __shared__ __attribute__((aligned(16))) float s_at[kMergeRC][64];  // A[k0 + k][j0 + j]
  __shared__ __attribute__((aligned(16))) float s_b[kMergeRC][64];   // B[j0 + j][n0 + n]
  const int tid = threadIdx.x;
  const int64_t n0 = (int64_t)blockIdx.y * 64, k0 = (int64_t)blockIdx.x * 64;
  const int rp = tid >> 3, cr = tid & 7;
  const int64_t k = k0 + 8 * cr;
  if (tid < 16) s_lv[tid] = cb.lv[tid];

  float acc[2][8];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.0f;

  for (int j0 = 0; j0 < r; j0 += kMergeRC) {
    const int jn = min(kMergeRC, r - j0);
    __syncthreads();  // the previous chunk is consumed
    for (int i = tid; i < kMergeRC * 64; i += 256) {
      const int j = i >> 6, c = i & 63;
      const int64_t kk = k0 + c, nn = n0 + c;
      s_at[j][c] = (j < jn) ? bf16_to_f32(A[kk * r + j0 + j]) : 0.0f;
      s_b[j][c] = (j < jn && nn < N) ? bf16_to_f32(B[(int64_t)(j0 + j) * N + nn]) : 0.0f;
    }
    __syncthreads();
    for (int j = 0; j < jn; ++j) {
      const floatx4 a0 = *reinterpret_cast<const floatx4*>(&s_at[j][8 * cr]);
      const floatx4 a1 = *reinterpret_cast<const floatx4*>(&s_at[j][8 * cr + 4]);
      const float b0 = s_b[j][2 * rp], b1 = s_b[j][2 * rp + 1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[0][e] = __builtin_fmaf(a0[e], b0, acc[0][e]);
        acc[0][e + 4] = __builtin_fmaf(a1[e], b0, acc[0][e + 4]);
        acc[1][e] = __builtin_fmaf(a0[e], b1, acc[1][e]);
        acc[1][e + 4] = __builtin_fmaf(a1[e], b1, acc[1][e + 4]);
      }
    }
  }
  __syncthreads();  // s_lv (written before the rank loop) is visible
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t n = n0 + 2 * rp + h;
    if (n >= N) continue;
    const int64_t e0 = n * K + k;                       // first of 8 elements, one block
    const uint32_t word = *reinterpret_cast<const uint32_t*>(codes + e0 / 2);
    const int64_t b = e0 / kBlock;
    const float cs = !absmax_q ? absmax_s2[b]
                     : cb.dq_fp8 ? block_scale_fp8(absmax_q[b], absmax_s2[b / kGroup])
                                 : block_scale(absmax_q[b], absmax_s2[b / kGroup]);
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const float w0 = s_lv[(word >> (4 * e)) & 15u] * cs;
      const float w1 = s_lv[(word >> (4 * e + 4)) & 15u] * cs;
      const float t0 = s * acc[h][e], t1 = s * acc[h][e + 1];
      o[e / 2] = pack_bf16x2(w0 + t0, w1 + t1);
    }
    *reinterpret_cast<u32x4*>(out + e0) = o;
  }
}

hipError_t launch_nf4_merge(Nf4Weight W, int64_t N, int64_t K, const uint16_t* A,
                            const uint16_t* B, int r, float scale, uint16_t* out,
                            hipStream_t stream) {
  dim3 grid((unsigned)(K / 64), (unsigned)((N + 63) / 64));
  hipLaunchKernelGGL(nf4_merge_kernel, grid, dim3(256), 0, stream, W.codes, W.absmax_q,
                     W.absmax_s2, N, K, A, B, r, scale, out, codebook_of(W));
  return hipGetLastError();
}

hipError_t launch_nf4_dequantize(Nf4Weight W, int64_t numel, void* out, bool bf16,
                                 hipStream_t stream) {
  const int64_t nwords = (numel + 7) / 8;
  int64_t blocks = (nwords + 511) / 512;  // two words per thread
  if (blocks > 65536) blocks = 65536;
  if (bf16)
    hipLaunchKernelGGL(nf4_dequantize_kernel<true>, dim3((unsigned)blocks), dim3(256), 0,
                       stream, W.codes, W.absmax_q, W.absmax_s2, numel, out, codebook_of(W));
  else
    hipLaunchKernelGGL(nf4_dequantize_kernel<false>, dim3((unsigned)blocks), dim3(256), 0,
                       stream, W.codes, W.absmax_q, W.absmax_s2, numel, out, codebook_of(W));
  return hipGetLastError();
}

}  // namespace qlora
