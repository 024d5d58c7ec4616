// Small-M forward (M <= 16): the decode-shaped product, bound by HBM.
//
//   Y = X bf16(W')^T + (s T) B          (ozercemkelahmet.com "QLoRA",
//                                        How it works, Step 5)
//
// The weight stream dominates: 0.5 byte of codes per weight plus one 8-bit
// constant per 64 weights. A wave owns 16 weight rows; each lane reads one
// 16-byte packet of codes (32 consecutive k of one row, inside one 64-block)
// per 128-wide k chunk, so a wave's load touches 16 rows x 64 contiguous
// bytes. The packet is dequantized in registers (level table in LDS, the
// double-dequantized block constant in one register) straight into the B
// operand of v_mfma_f32_16x16x32_bf16, with the tokens as the A operand
// (rows >= M are zero). The contraction index inside one MFMA is permuted
// identically for both operands, which leaves the sum unchanged.
//
// The K range is split across the grid's y dimension; the last split also
// accumulates the adapter columns (s T) B. With more than one split, float32
// partials are summed in a fixed order by a second small kernel, so results
// are deterministic.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace qlora {

namespace {

constexpr int kRowsPerBlock = 64;  // 4 waves x 16 rows
constexpr int kChunk = 128;        // k per iteration per wave

__device__ __forceinline__ bf16x8 dequant8(uint32_t word, float cs, const float* lv) {
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float lo = lv[(word >> (8 * j)) & 15u] * cs;
    const float hi = lv[(word >> (8 * j + 4)) & 15u] * cs;
    o[j] = pack_bf16x2(lo, hi);
  }
  return as_bf16x8(o);
}

__global__ void __launch_bounds__(256)
nf4_gemv_kernel(const uint16_t* __restrict__ X, const uint8_t* __restrict__ codes,
                const uint8_t* __restrict__ absmax_q, const float* __restrict__ absmax_s2,
                const uint16_t* __restrict__ sT, int64_t ldt, const uint16_t* __restrict__ B,
                int M, int64_t N, int64_t K, int r, int64_t kchunk,
                uint16_t* __restrict__ Y, float* __restrict__ part) {
#pragma clang fp contract(off)
  __shared__ float s_lv[16];
  const int tid = threadIdx.x;
  if (tid < 16) s_lv[tid] = kNF4[tid];
  __syncthreads();

  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int64_t n = (int64_t)blockIdx.x * kRowsPerBlock + wave * 16 + col;
  const bool nvalid = n < N;
  const int ks = blockIdx.y, nsplit = gridDim.y;
  const int64_t kbeg = (int64_t)ks * kchunk;
  const int64_t kend = std::min<int64_t>(K, kbeg + kchunk);
  const int m = col;  // token row of this lane's A fragment
  const bool mvalid = m < M;

  floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const uint8_t* wrow = codes + (nvalid ? n : 0) * (K / 2);
  const uint16_t* xrow = X + (int64_t)(mvalid ? m : 0) * K;

  for (int64_t k0 = kbeg; k0 < kend; k0 += kChunk) {
    const int64_t kb = k0 + 32 * g;
    const bool kvalid = kb < kend;  // kend and kb are multiples of 32
    u32x4 c = {0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u};
    float cs = 0.0f;
    if (nvalid && kvalid) {
      c = *reinterpret_cast<const u32x4*>(wrow + kb / 2);
      const int64_t b = (n * K + kb) / kBlock;
      cs = block_scale(absmax_q[b], absmax_s2[b / kGroup]);
    }
    u32x4 xv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (mvalid && kvalid)
        xv[j] = *reinterpret_cast<const u32x4*>(xrow + kb + 8 * j);
      else
        xv[j] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xv[j]), dequant8(c[j], cs, s_lv),
                                                    acc, 0, 0, 0);
  }

  // adapter columns: sum_j (sT)[m][j] B[j][n], in the last split
  if (ks == nsplit - 1) {
    for (int j0 = 0; j0 < r; j0 += 32) {
      const int jj = j0 + 8 * g;
      u32x4 xa = {0u, 0u, 0u, 0u};
      if (mvalid) xa = *reinterpret_cast<const u32x4*>(sT + (int64_t)m * ldt + jj);
      u32x4 wb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j1 = jj + 2 * e, j2 = j1 + 1;
        const uint32_t lo = (nvalid && j1 < r) ? B[(int64_t)j1 * N + n] : 0u;
        const uint32_t hi = (nvalid && j2 < r) ? B[(int64_t)j2 * N + n] : 0u;
        wb[e] = lo | (hi << 16);
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa), as_bf16x8(wb), acc, 0, 0, 0);
    }
  }

  // D[i][j]: lane holds rows i = 4 g + v (tokens), column j = col (weight row)
  if (nvalid) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int mm = 4 * g + v;
      if (mm < M) {
        if (nsplit == 1)
          Y[(int64_t)mm * N + n] = (uint16_t)(pack_bf16x2(acc[v], 0.0f) & 0xffffu);
        else
          part[((int64_t)ks * M + mm) * N + n] = acc[v];
      }
    }
  }
}

__global__ void gemv_reduce_kernel(const float* __restrict__ part, int splits, int M, int64_t N,
                                   uint16_t* __restrict__ Y) {
  const int64_t total = (int64_t)M * N;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    float v = 0.0f;
    for (int s = 0; s < splits; ++s) v += part[(int64_t)s * total + i];
    Y[i] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xffffu);
  }
}

// K is split into chunks of whole 128-wide iterations (the last may be 64).
int64_t gemv_kchunk(int64_t N, int64_t K) {
  const int64_t tiles = (N + kRowsPerBlock - 1) / kRowsPerBlock;
  int64_t splits = std::max<int64_t>(1, 512 / std::max<int64_t>(tiles, 1));
  const int64_t iters = (K + kChunk - 1) / kChunk;
  splits = std::min(splits, std::max<int64_t>(1, iters / 2));
  const int64_t per = (iters + splits - 1) / splits;
  return per * kChunk;
}

}  // namespace

int64_t gemv_partial_elems(int64_t M, int64_t N, int64_t K) {
  if (M > kGemvMaxM) return 0;
  const int64_t kc = gemv_kchunk(N, K);
  const int64_t splits = (K + kc - 1) / kc;
  return splits > 1 ? splits * M * N : 0;
}

size_t ws_offset_part(int64_t M, int64_t N, int64_t K, int r);
size_t ws_offset_st(int64_t M, int64_t N, int64_t K, int r);
hipError_t launch_compute_T(const uint16_t* X, const uint16_t* A, int64_t M, int64_t N, int64_t K,
                            int r, float scale, float* out32, void* ws, hipStream_t stream);

hipError_t launch_fwd_gemv(const uint16_t* X, Nf4Weight W, const uint16_t* A, const uint16_t* B,
                           int M, int64_t N, int64_t K, int r, float scale, uint16_t* Y,
                           float* T_out, void* ws_, hipStream_t stream, hipEvent_t ev0,
                           hipEvent_t ev1) {
  char* ws = reinterpret_cast<char*>(ws_);
  hipError_t e = launch_compute_T(X, A, M, N, K, r, scale, T_out, ws_, stream);
  if (e != hipSuccess) return e;
  const int64_t r64 = (r + 63) / 64 * 64;
  const uint16_t* sT = reinterpret_cast<const uint16_t*>(ws + ws_offset_st(M, N, K, r));
  float* part = reinterpret_cast<float*>(ws + ws_offset_part(M, N, K, r));
  const int64_t kc = gemv_kchunk(N, K);
  const int splits = (int)((K + kc - 1) / kc);
  dim3 grid((unsigned)((N + kRowsPerBlock - 1) / kRowsPerBlock), (unsigned)splits);
  e = record_if(ev0, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(nf4_gemv_kernel, grid, dim3(256), 0, stream, X, W.codes, W.absmax_q,
                     W.absmax_s2, sT, r64, B, M, N, K, r, kc, Y, part);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = record_if(ev1, stream);
  if (e != hipSuccess || splits == 1) return e;
  const int64_t total = (int64_t)M * N;
  unsigned blocks = (unsigned)std::min<int64_t>(4096, (total + 255) / 256);
  hipLaunchKernelGGL(gemv_reduce_kernel, dim3(blocks), dim3(256), 0, stream, part, splits, M, N, Y);
  return hipGetLastError();
}

}  // namespace qlora
