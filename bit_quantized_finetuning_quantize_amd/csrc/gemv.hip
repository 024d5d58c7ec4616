// Small-M forward (M <= 16): the decode-shaped product, bound by HBM.
//
//   Y = X bf16(W')^T + s (X A) B          (ozercemkelahmet.com "QLoRA",
//                                          How it works, Step 5)
//
// Two launches per call.
//
// 1. nf4_gemv_main. The grid's x dimension holds two kinds of workgroups.
//    GEMV workgroups (one per 64 weight rows and K split) stream the NF4
//    store: a wave owns 16 rows; each lane issues, before any arithmetic,
//    all of its 16-byte code packets (32 consecutive k of one row, inside
//    one 64-block) and the few dword loads that hold their 8-bit and
//    second-level constants, while the workgroup stages the split's token
//    rows in LDS; then it dequantizes each packet in registers
//    (level table and fl(q8/255) table in LDS) straight into the B operand
//    of v_mfma_f32_16x16x32_bf16, with the tokens as the A operand (rows
//    >= M are zero). The contraction index inside one MFMA is permuted
//    identically for both operands, which leaves the sum unchanged.
//    Adapter workgroups (one per 128-wide k chunk and 64 adapter columns)
//    compute the chunk's partial of T = X A at the same time, staging A
//    through LDS to transpose it into MFMA operands.
// 2. nf4_gemv_epilogue sums the float32 partials of Y and T in a fixed order
//    (deterministic), adds s T B in float32 and rounds Y to bf16.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace qlora {

namespace {

constexpr int kRowsPerBlock = 64;  // 4 waves x 16 rows
constexpr int kChunk = 128;        // k per iteration per wave
constexpr int kTCols = 64;         // adapter columns per adapter workgroup

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* base, int64_t bytes) {
  if (bytes > 0x7ffffff0LL) bytes = 0x7ffffff0LL;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ bf16x8 dequant8(uint32_t word, float cs, const float* lv) {
#pragma clang fp contract(off)
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float lo = lv[(word >> (8 * j)) & 15u] * cs;
    const float hi = lv[(word >> (8 * j + 4)) & 15u] * cs;
    o[j] = pack_bf16x2(lo, hi);
  }
  return as_bf16x8(o);
}

struct GemvArgs {
  const uint16_t* X;
  const uint8_t* codes;
  const uint8_t* absmax_q;
  const float* absmax_s2;
  const uint16_t* A;
  int M, r;
  int64_t N, K;
  int64_t kchunk;  // I * 128
  int ntiles;      // GEMV workgroups per split
  int splits;      // K splits of the GEMV workgroups
  int tblocks;     // 64-column groups of the adapter
  float* part_y;   // [splits][M][N]
  float* part_t;   // [ceil(K/128)][M][r]
};

// GEMV workgroup: weight rows [64 tile, 64 tile + 64), K split ks. The
// token rows of the split (M x kchunk bf16) are staged once in LDS; each
// lane then issues all of its code packets plus the few loads that cover
// its block constants before any arithmetic.
template <int I>
__device__ void gemv_tile(const GemvArgs& a, int tile, int ks, const float* lv, const float* l8,
                          uint16_t* sX) {
#pragma clang fp contract(off)
  constexpr int kOut = 0x7ffffff0;  // any offset past every range: loads return 0
  constexpr int kc = I * kChunk;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int64_t n = (int64_t)tile * kRowsPerBlock + wave * 16 + col;
  const int64_t kbeg = (int64_t)ks * kc;
  const int64_t kend = std::min<int64_t>(a.K, kbeg + kc);
  const int m = col;

  const __amdgpu_buffer_rsrc_t rc = rsrc_of(a.codes, a.N * a.K / 2);
  const __amdgpu_buffer_rsrc_t rq = rsrc_of(a.absmax_q, a.N * a.K / kBlock);
  const __amdgpu_buffer_rsrc_t rs = rsrc_of(a.absmax_s2, (a.N * a.K / kBlock + kGroup - 1) / kGroup * 4);
  const __amdgpu_buffer_rsrc_t rx = rsrc_of(a.X, (int64_t)a.M * a.K * 2);

  // codes: one 16-byte packet per iteration
  u32x4 c[I];
  const bool nok = n < a.N;
  const int64_t e0 = n * a.K + kbeg + 32 * g;  // element of this lane's first packet
#pragma unroll
  for (int i = 0; i < I; ++i) {
    const bool ok = nok && kbeg + i * kChunk + 32 * g < kend;
    c[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                         rc, ok ? (int)((e0 + i * kChunk) / 2) : kOut, 0, 0));
  }
  // 8-bit constants: packet i lies in block b0 + 2 i; one dword covers 4 blocks
  const int64_t b0 = e0 / kBlock;
  uint32_t qw[(2 * I + 3) / 4 + 1];
#pragma unroll
  for (int w = 0; w < (2 * I + 3) / 4 + 1; ++w) {
    const int64_t bb = (b0 & ~3LL) + 4 * w;
    qw[w] = nok ? __builtin_amdgcn_raw_buffer_load_b32(rq, (int)bb, 0, 0) : 0u;
  }
  // second-level constants: blocks b0 .. b0 + 2I - 2 span at most two groups
  const int64_t g0 = b0 / kGroup;
  const float s2a = __builtin_bit_cast(
      float, __builtin_amdgcn_raw_buffer_load_b32(rs, nok ? (int)(g0 * 4) : kOut, 0, 0));
  const float s2b = __builtin_bit_cast(
      float, __builtin_amdgcn_raw_buffer_load_b32(rs, nok ? (int)((g0 + 1) * 4) : kOut, 0, 0));
  // token rows of the split -> LDS [M][kc] (k >= kend is 0)
  {
    const int units = a.M * (kc / 8);  // 16-byte units
    for (int u = tid; u < units; u += 256) {
      const int mm = u / (kc / 8), k8 = (u % (kc / 8)) * 8;
      const int64_t k = kbeg + k8;
      const bool ok = k < kend;
      const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    rx, ok ? (int)(((int64_t)mm * a.K + k) * 2) : kOut,
                                                    0, 0));
      *reinterpret_cast<u32x4*>(&sX[mm * kc + k8]) = v;
    }
  }
  __syncthreads();

  floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < I; ++i) {
    const int64_t b = b0 + 2 * i;
    const int qi = (int)(b - (b0 & ~3LL));
    const uint32_t q8 = (qw[qi >> 2] >> (8 * (qi & 3))) & 0xffu;
    const float s2 = (b / kGroup == g0) ? s2a : s2b;
    const float cs = l8[q8] * s2;
    const int kl = i * kChunk + 32 * g;  // this lane's k inside the split
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 xv = {0u, 0u, 0u, 0u};  // token rows >= M are zero
      if (m < a.M) xv = *reinterpret_cast<const u32x4*>(&sX[m * kc + kl + 8 * j]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xv), dequant8(c[i][j], cs, lv), acc,
                                                    0, 0, 0);
    }
  }
  // D[i][j]: lane holds rows i = 4 g + v (tokens), column j = col (weight row)
  if (nok) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int mm = 4 * g + v;
      if (mm < a.M) a.part_y[((int64_t)ks * a.M + mm) * a.N + n] = acc[v];
    }
  }
}

// A chunk (4 x 16 bytes per thread) and token fragments of one adapter chunk.
struct AdapterChunk {
  u32x4 a[4];   // 4 x 16 bytes of A (eight columns each)
  u32x4 x[4];   // token fragments of the 4 MFMA steps
};

__device__ __forceinline__ void adapter_load(const GemvArgs& a, int64_t k0, int64_t kend, int j0,
                                             AdapterChunk& c) {
  constexpr int kOut = 0x7ffffff0;
  const int tid = threadIdx.x;
  const int lane = tid & 63, g = (lane >> 4), m = lane & 15;
  const __amdgpu_buffer_rsrc_t ra = rsrc_of(a.A, a.K * a.r * 2);
  const __amdgpu_buffer_rsrc_t rx = rsrc_of(a.X, (int64_t)a.M * a.K * 2);
  if ((a.r & 7) == 0) {  // rows of A hold whole groups of eight columns
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + u * 256;  // 128 rows x 8 column groups
      const int kk = e >> 3, j = j0 + (e & 7) * 8;
      const int64_t k = k0 + kk;
      const bool ok = k < kend && j < a.r;
      c.a[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             ra, ok ? (int)((k * a.r + j) * 2) : kOut, 0, 0));
    }
  } else {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + u * 256;
      const int kk = e >> 3, j = j0 + (e & 7) * 8;
      const int64_t k = k0 + kk;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        uint32_t w = 0;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int jj = j + 2 * h + b;
          const bool ok = k < kend && jj < a.r;
          const uint32_t v = __builtin_amdgcn_raw_buffer_load_b16(
              ra, ok ? (int)((k * a.r + jj) * 2) : kOut, 0, 0);
          w |= (v & 0xffffu) << (16 * b);
        }
        c.a[u][h] = w;
      }
    }
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int64_t kb = k0 + s * 32 + 8 * g;
    c.x[s] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                   rx, (m < a.M && kb < kend) ? (int)(((int64_t)m * a.K + kb) * 2) : kOut, 0, 0));
  }
}

// Adapter workgroup: the partial of T over one 128-wide k chunk for
// adapter columns [64 t, 64 t + 64); wave w owns 16 of them. The chunk of A
// is staged through LDS so that each lane can read 8 consecutive k of one
// column. One workgroup per chunk keeps every load of the adapter product in
// flight at once.
__device__ void adapter_tile(const GemvArgs& a, int chunk, int t, uint16_t* sA) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int64_t k0 = (int64_t)chunk * kChunk;
  const int64_t kend = std::min<int64_t>(a.K, k0 + kChunk);
  const int j0 = t * kTCols;
  AdapterChunk cur;
  adapter_load(a, k0, kend, j0, cur);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = tid + u * 256;
    *reinterpret_cast<u32x4*>(&sA[(e >> 3) * kTCols + (e & 7) * 8]) = cur.a[u];
  }
  __syncthreads();
  floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < kChunk / 32; ++s) {
    const int kl = s * 32 + 8 * g;  // this lane's 8 k inside the chunk
    u32x4 wb;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = sA[(kl + 2 * e) * kTCols + wave * 16 + col];
      const uint32_t hi = sA[(kl + 2 * e + 1) * kTCols + wave * 16 + col];
      wb[e] = lo | (hi << 16);
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(cur.x[s]), as_bf16x8(wb), acc, 0, 0, 0);
  }
  const int j = j0 + wave * 16 + col;
  if (j < a.r) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int mm = 4 * g + v;
      if (mm < a.M) a.part_t[((int64_t)chunk * a.M + mm) * a.r + j] = acc[v];
    }
  }
}

template <int I>
__global__ void __launch_bounds__(256) nf4_gemv_main(GemvArgs a) {
  __shared__ float s_lv[16];
  __shared__ float s_l8[256];
  // adapter A chunk [128][64] or token rows [16][I * 128], never both
  __shared__ __attribute__((aligned(16))) uint16_t s_a[(kChunk * kTCols > 16 * I * kChunk)
                                                           ? kChunk * kTCols
                                                           : 16 * I * kChunk];
  const int tid = threadIdx.x;
  if (tid < 16) s_lv[tid] = kNF4[tid];
  {
#pragma clang fp contract(off)
    s_l8[tid] = static_cast<float>(tid) / 255.0f;  // IEEE division
  }
  __syncthreads();
  const int id = blockIdx.x;
  const int ngemv = a.ntiles * a.splits;
  if (id < ngemv) {
    gemv_tile<I>(a, id % a.ntiles, id / a.ntiles, s_lv, s_l8, s_a);
  } else {
    const int u = id - ngemv;
    adapter_tile(a, u / a.tblocks, u % a.tblocks, s_a);
  }
}

// Y[m][n] = bf16( sum_s Py[s][m][n] + s * sum_j T[m][j] B[j][n] ),
// T = sum_c Pt[c] (fixed order). Workgroup: 64 columns x all tokens. The
// partial sums are loaded eight at a time so their latencies overlap.
__global__ void __launch_bounds__(256)
nf4_gemv_epilogue(const float* __restrict__ part_y, const float* __restrict__ part_t,
                  int splits, int tsplits, int M, int64_t N, int r, const uint16_t* __restrict__ B,
                  float scale, uint16_t* __restrict__ Y, float* __restrict__ T_out) {
  extern __shared__ float s_t[];  // [M][r]
  const int tid = threadIdx.x;
  for (int e = tid; e < M * r; e += 256) {
    float v = 0.0f;
    int s = 0;
    for (; s + 8 <= tsplits; s += 8) {
      float t[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) t[u] = part_t[(int64_t)(s + u) * M * r + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) v += t[u];
    }
    for (; s < tsplits; ++s) v += part_t[(int64_t)s * M * r + e];
    s_t[e] = v;
    if (T_out && blockIdx.x == 0) T_out[e] = v;
  }
  __syncthreads();
  const int64_t n = (int64_t)blockIdx.x * 64 + (tid & 63);
  if (n >= N) return;
  for (int m = tid >> 6; m < M; m += 4) {
    float y = 0.0f;
    int s = 0;
    for (; s + 8 <= splits; s += 8) {
      float t[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) t[u] = part_y[((int64_t)(s + u) * M + m) * N + n];
#pragma unroll
      for (int u = 0; u < 8; ++u) y += t[u];
    }
    for (; s < splits; ++s) y += part_y[((int64_t)s * M + m) * N + n];
    float l = 0.0f;
    int j = 0;
    for (; j + 8 <= r; j += 8) {
      float bv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) bv[u] = bf16_to_f32(B[(int64_t)(j + u) * N + n]);
#pragma unroll
      for (int u = 0; u < 8; ++u) l += s_t[m * r + j + u] * bv[u];
    }
    for (; j < r; ++j) l += s_t[m * r + j] * bf16_to_f32(B[(int64_t)j * N + n]);
    y += scale * l;
    Y[(int64_t)m * N + n] = (uint16_t)(pack_bf16x2(y, 0.0f) & 0xffffu);
  }
}

// iterations per wave per split: fewer token rows leave room for deeper
// prefetch
int gemv_iters(int M) { return M <= 4 ? 8 : 4; }

}  // namespace

int64_t gemv_splits(int64_t M, int64_t K) {
  const int64_t kc = (int64_t)gemv_iters((int)M) * kChunk;
  return (K + kc - 1) / kc;
}

int64_t gemv_partial_elems(int64_t M, int64_t N, int64_t K, int r) {
  if (M > kGemvMaxM) return 0;
  return gemv_splits(M, K) * M * N + (K + kChunk - 1) / kChunk * M * r;
}

size_t ws_offset_part(int64_t M, int64_t N, int64_t K, int r);

hipError_t launch_fwd_gemv(const uint16_t* X, Nf4Weight W, const uint16_t* A, const uint16_t* B,
                           int M, int64_t N, int64_t K, int r, float scale, uint16_t* Y,
                           float* T_out, void* ws_, hipStream_t stream, hipEvent_t ev0,
                           hipEvent_t ev1) {
  char* ws = reinterpret_cast<char*>(ws_);
  const int I = gemv_iters(M);
  const int splits = (int)gemv_splits(M, K);
  float* part_y = reinterpret_cast<float*>(ws + ws_offset_part(M, N, K, r));
  float* part_t = part_y + (int64_t)splits * M * N;
  const int tblocks = (r + kTCols - 1) / kTCols;
  const int nchunks = (int)((K + kChunk - 1) / kChunk);
  GemvArgs a{X, W.codes, W.absmax_q, W.absmax_s2, A, M, r, N, K, (int64_t)I * kChunk,
             (int)((N + kRowsPerBlock - 1) / kRowsPerBlock), splits, tblocks, part_y, part_t};
  dim3 grid((unsigned)(a.ntiles * splits + nchunks * tblocks));
  hipError_t e = record_if(ev0, stream);
  if (e != hipSuccess) return e;
  if (I == 8)
    hipLaunchKernelGGL(nf4_gemv_main<8>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(nf4_gemv_main<4>, grid, dim3(256), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = record_if(ev1, stream);
  if (e != hipSuccess) return e;
  const size_t lds = (size_t)M * r * sizeof(float);
  hipLaunchKernelGGL(nf4_gemv_epilogue, dim3((unsigned)((N + 63) / 64)), dim3(256), lds, stream,
                     part_y, part_t, splits, nchunks, M, N, r, B, scale, Y, T_out);
  return hipGetLastError();
}

}  // namespace qlora
