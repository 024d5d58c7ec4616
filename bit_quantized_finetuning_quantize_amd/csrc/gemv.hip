// Small-M forward (M <= 16): the decode-shaped product, bound by HBM.
//
//   Y = X bf16(W')^T + s (X A) B          (ozercemkelahmet.com "QLoRA",
//                                          How it works, Step 5)
//
// Two launches per call.
//
// 1. nf4_gemv_main. The grid's x dimension holds two kinds of workgroups of
//    kKQ x 4 waves. Adapter workgroups come first (one per kKQ x 128 k and
//    64 adapter columns) and compute partials of T = X A, staging A through
//    LDS to transpose it into MFMA operands. GEMV workgroups (one per 64
//    weight rows and K split) stream the NF4 store: wave w owns 16 rows
//    (w % 4) and one of kKQ k groups of the split (w / 4). Each lane issues,
//    before any arithmetic, all of its 16-byte code packets (32 consecutive
//    k of one row, inside one 64-block) and the few dword loads that hold
//    their 8-bit and second-level constants, while the workgroup stages the
//    split's token rows in LDS. It then dequantizes each packet in registers
//    (v_perm_b32 byte selection from the block's 16 possible weights, the
//    fl(q8/255) table in LDS) straight into the B
//    operand of v_mfma_f32_16x16x32_bf16, with the tokens as the A operand
//    (rows >= M are zero). The contraction index inside one MFMA is permuted
//    identically for both operands, which leaves the sum unchanged. The k
//    groups are summed through LDS in a fixed order.
// 2. nf4_gemv_epilogue sums the float32 partials of Y and T in a fixed order
//    (deterministic), adds s T B in float32 and rounds Y to bf16.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace qlora {

namespace {

#ifndef QLORA_GEMV_KQ
#define QLORA_GEMV_KQ 2
#endif
constexpr int kKQ = QLORA_GEMV_KQ;  // k groups per workgroup (4 waves each)
constexpr int kThreads = 256 * kKQ;
constexpr int kRowsPerBlock = 64;   // 4 row groups x 16 rows
constexpr int kChunk = 128;         // k per packet column of a wave
constexpr int kTK = kChunk * kKQ;   // k per adapter workgroup
constexpr int kTCols = 64;          // adapter columns per adapter workgroup

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* base, int64_t bytes) {
  if (bytes > 0x7ffffff0LL) bytes = 0x7ffffff0LL;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

struct GemvArgs {
  const uint16_t* X;
  const uint8_t* codes;
  const uint8_t* absmax_q;
  const float* absmax_s2;
  const uint16_t* A;
  int M, r;
  int64_t N, K;
  int ntiles;      // GEMV workgroups per split
  int splits;      // K splits of the GEMV workgroups
  int tchunks;     // 512-wide k chunks of the adapter product
  int tblocks;     // 64-column groups of the adapter
  float* part_y;   // [splits][M][N]
  float* part_t;   // [tchunks][M][r]
};

// LDS of one workgroup, reused by the three phases that need it.
template <int I>
struct alignas(16) Shared {
  static constexpr int kX = 16 * I * kChunk;   // token rows [16][kc] bf16
  static constexpr int kA = kTK * kTCols;      // adapter chunk [512][64] bf16
  static constexpr int kU16 = kX > kA ? kX : kA;
  float l8[256];
  union {
    uint16_t x[kU16];
    floatx4 red[4 * kKQ][64];  // per-wave accumulators for the workgroup reduction
  };
};

// GEMV workgroup: weight rows [64 tile, 64 tile + 64), K split ks of kc =
// I*128. kDQ false: the store has no 8-bit codes and absmax_s2 holds one
// float32 constant per block (one dword load per packet). Wave w owns 16 rows (row group w & 3) and one of the kKQ k groups
// of the split (w >> 2); the groups are summed in a fixed order through LDS.
// The split's token rows are staged once in LDS; every global load is
// issued before any arithmetic.
template <int I, bool kDQ>
__device__ void gemv_tile(const GemvArgs& a, int tile, int ks, Shared<I>& sh) {
#pragma clang fp contract(off)
  constexpr int kOut = 0x7ffffff0;  // an offset past every range: the load returns 0
  constexpr int kc = I * kChunk;
  constexpr int P = I / kKQ;        // packets per lane
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, g = lane >> 4;
  const int rg = wave & 3, kq = wave >> 2;
  const int64_t n = (int64_t)tile * kRowsPerBlock + rg * 16 + col;
  const int64_t kbeg = (int64_t)ks * kc;
  const int64_t kend = std::min<int64_t>(a.K, kbeg + kc);
  const int kw = kq * (kc / kKQ);   // this wave's first k inside the split

  const __amdgpu_buffer_rsrc_t rc = rsrc_of(a.codes, a.N * a.K / 2);
  const __amdgpu_buffer_rsrc_t rq = rsrc_of(a.absmax_q, kDQ ? a.N * a.K / kBlock : 0);
  const __amdgpu_buffer_rsrc_t rs =
      rsrc_of(a.absmax_s2, kDQ ? (a.N * a.K / kBlock + kGroup - 1) / kGroup * 4
                               : a.N * a.K / kBlock * 4);
  const __amdgpu_buffer_rsrc_t rx = rsrc_of(a.X, (int64_t)a.M * a.K * 2);

  // Every load is unconditional (an invalid one reads past the range and
  // returns 0), so no wait covers a load that is not needed yet. The token
  // rows go first: waiting for them then does not wait for the weights.
  // A wave's units lie in one token row (kc / 8 >= 64): rows >= M are not
  // loaded at all (a wave-uniform branch) and stored as zeros.
  constexpr int kXU = 16 * kc / 8 / kThreads;  // 16-byte units per thread
  static_assert(kc / 8 >= 64, "a wave's token units must lie in one row");
  u32x4 xr[kXU];
#pragma unroll
  for (int j = 0; j < kXU; ++j) {
    const int mm = (wave * 64 + kThreads * j) / (kc / 8);  // wave-uniform
    xr[j] = u32x4{0u, 0u, 0u, 0u};
    if (mm < a.M) {
      const int k8 = ((tid + kThreads * j) % (kc / 8)) * 8;
      const bool ok = kbeg + k8 < kend;
      const uint32_t off = ((uint32_t)mm * (uint32_t)a.K + (uint32_t)(kbeg + k8)) * 2u;
      xr[j] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, ok ? (int)off : kOut, 0, 0));
    }
  }
  // codes: packet p = 32 consecutive k of row n at kw + 128 p + 32 g
  const bool nok = n < a.N;
  const int64_t e0 = n * a.K + kbeg + kw + 32 * g;
  u32x4 c[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const bool ok = nok && kbeg + kw + p * kChunk + 32 * g < kend;
    c[p] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                         rc, ok ? (int)((e0 + p * kChunk) / 2) : kOut, 0, 0));
  }
  // 8-bit constants: packet p lies in block b0 + 2 p; one dword holds 4 blocks
  const int64_t b0 = e0 / kBlock;
  constexpr int kQW = (2 * P + 1) / 4 + 1;
  uint32_t qw[kQW];
  float s2a = 0.0f, s2b = 0.0f;
  const int64_t g0 = b0 / kGroup;
  float cb[P];  // without double quantization: each packet's block constant
  if constexpr (kDQ) {
#pragma unroll
    for (int w = 0; w < kQW; ++w)
      qw[w] = __builtin_amdgcn_raw_buffer_load_b32(rq, nok ? (int)((b0 & ~3LL) + 4 * w) : kOut, 0, 0);
    // second-level constants: blocks b0 .. b0 + 2P - 2 span at most two groups
    s2a = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(rs, nok ? (int)(g0 * 4) : kOut, 0, 0));
    s2b = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(rs, nok ? (int)((g0 + 1) * 4) : kOut, 0, 0));
  } else {
#pragma unroll
    for (int p = 0; p < P; ++p)
      cb[p] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(rs, nok ? (int)((b0 + 2 * p) * 4) : kOut, 0, 0));
  }
  // lookup tables, built while the loads are in flight
  if (tid < 256) {
#pragma clang fp contract(off)
    sh.l8[tid] = static_cast<float>(tid) / 255.0f;  // IEEE division
  }
  // all 16 rows are stored (rows >= M are zeros), so the reads need no branch
#pragma unroll
  for (int j = 0; j < kXU; ++j) {
    const int u = tid + kThreads * j;
    *reinterpret_cast<u32x4*>(&sh.x[(u / (kc / 8)) * kc + (u % (kc / 8)) * 8]) = xr[j];
  }
  __syncthreads();

  floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int p = 0; p < P; ++p) {
    float cs;
    if constexpr (kDQ) {
      const int64_t b = b0 + 2 * p;
      const int qi = (int)(b - (b0 & ~3LL));
      const uint32_t q8 = (qw[qi >> 2] >> (8 * (qi & 3))) & 0xffu;
      const float s2 = (b / kGroup == g0) ? s2a : s2b;
      cs = sh.l8[q8] * s2;
    } else {
      cs = cb[p];
    }
    const int kl = kw + p * kChunk + 32 * g;  // this lane's k inside the split
    const PermTable pt = perm_table(cs);  // lookups by v_perm: no LDS round trips
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // MFMA j takes elements 8j..8j+7 of every lane's packet, for the token
      // operand and the weight operand alike: the sum over k is unchanged
      const u32x4 xv = *reinterpret_cast<const u32x4*>(&sh.x[col * kc + kl + 8 * j]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xv),
                                                    as_bf16x8(dequant_word_perm(c[p][j], pt)),
                                                    acc, 0, 0, 0);
    }
  }
  __syncthreads();  // the token rows are dead: their LDS takes the reduction
  sh.red[wave][lane] = acc;
  __syncthreads();
  if (kq == 0 && nok) {
    floatx4 t = sh.red[rg][lane];
#pragma unroll
    for (int q = 1; q < kKQ; ++q) {
      const floatx4 u = sh.red[rg + 4 * q][lane];
#pragma unroll
      for (int v = 0; v < 4; ++v) t[v] += u[v];
    }
    // D[i][j]: this lane holds tokens i = 4 g + v of weight row j = col
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int mm = 4 * g + v;
      if (mm < a.M) a.part_y[((int64_t)ks * a.M + mm) * a.N + n] = t[v];
    }
  }
}

// Adapter workgroup: the partial of T = X A over one kTK-wide k chunk for
// adapter columns [64 t, 64 t + 64). Wave w owns 16 columns (w & 3) of one
// 128-wide part of the chunk (w >> 2); the parts are summed in a fixed
// order. A is staged through LDS so that a lane can read 8 consecutive k of
// one column.
template <int I>
__device__ void adapter_tile(const GemvArgs& a, int chunk, int t, Shared<I>& sh) {
  constexpr int kOut = 0x7ffffff0;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int cg = wave & 3, kq = wave >> 2;
  const int64_t k0 = (int64_t)chunk * kTK;
  const int64_t kend = std::min<int64_t>(a.K, k0 + kTK);
  const int j0 = t * kTCols;
  const __amdgpu_buffer_rsrc_t ra = rsrc_of(a.A, a.K * a.r * 2);
  const __amdgpu_buffer_rsrc_t rx = rsrc_of(a.X, (int64_t)a.M * a.K * 2);

  // token fragments of this wave's 4 MFMA steps (row col, k 8 g of each 32)
  u32x4 xf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int64_t kb = k0 + kq * kChunk + s * 32 + 8 * g;
    xf[s] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                   rx, (col < a.M && kb < kend) ? (int)(((int64_t)col * a.K + kb) * 2) : kOut, 0,
                   0));
  }
  // A chunk [512][64] -> LDS: thread loads 16-byte units (8 columns of a row)
  constexpr int kAU = kTK * kTCols / 8 / kThreads;  // 4 16-byte units per thread
  u32x4 av[kAU];
  if ((a.r & 7) == 0) {  // rows of A hold whole groups of eight columns
#pragma unroll
    for (int u = 0; u < kAU; ++u) {
      const int e = tid + u * kThreads;
      const int64_t k = k0 + (e >> 3);
      const int j = j0 + (e & 7) * 8;
      const bool ok = k < kend && j < a.r;
      av[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            ra, ok ? (int)((k * a.r + j) * 2) : kOut, 0, 0));
    }
  } else {
#pragma unroll
    for (int u = 0; u < kAU; ++u) {
      const int e = tid + u * kThreads;
      const int64_t k = k0 + (e >> 3);
      const int j = j0 + (e & 7) * 8;
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
        av[u][h] = w;
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kAU; ++u) {
    const int e = tid + u * kThreads;
    *reinterpret_cast<u32x4*>(&sh.x[(e >> 3) * kTCols + (e & 7) * 8]) = av[u];
  }
  __syncthreads();
  floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int kl = kq * kChunk + s * 32 + 8 * g;  // this lane's 8 k inside the chunk
    u32x4 wb;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = sh.x[(kl + 2 * e) * kTCols + cg * 16 + col];
      const uint32_t hi = sh.x[(kl + 2 * e + 1) * kTCols + cg * 16 + col];
      wb[e] = lo | (hi << 16);
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xf[s]), as_bf16x8(wb), acc, 0, 0, 0);
  }
  __syncthreads();
  sh.red[wave][lane] = acc;
  __syncthreads();
  const int j = j0 + cg * 16 + col;
  if (kq == 0 && j < a.r) {
    floatx4 tt = sh.red[cg][lane];
#pragma unroll
    for (int q = 1; q < kKQ; ++q) {
      const floatx4 u = sh.red[cg + 4 * q][lane];
#pragma unroll
      for (int v = 0; v < 4; ++v) tt[v] += u[v];
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int mm = 4 * g + v;
      if (mm < a.M) a.part_t[((int64_t)chunk * a.M + mm) * a.r + j] = tt[v];
    }
  }
}

// Adapter workgroups come first in the grid so that they start first.
template <int I, bool kDQ>
__global__ void __launch_bounds__(kThreads) nf4_gemv_main(GemvArgs a) {
  __shared__ Shared<I> sh;
  const int id = blockIdx.x;
  const int nadapt = a.tchunks * a.tblocks;
  if (id < nadapt)
    adapter_tile<I>(a, id / a.tblocks, id % a.tblocks, sh);
  else
    gemv_tile<I, kDQ>(a, (id - nadapt) % a.ntiles, (id - nadapt) / a.ntiles, sh);
}

// Y[m][n] = bf16( sum_s Py[s][m][n] + s * sum_j T[m][j] B[j][n] ),
// T = sum_c Pt[c] (fixed orders). Workgroup: 64 columns x all tokens.
// Thread: column n = n0 + tid % 64, tokens m = tid / 64 + 4 i. The first
// pass of every input (Y partials of YS splits, BU 16-byte units of the B
// tile, T partials of TS chunks for element tid) is issued before any of it
// is used, branch-free, so the shapes the pass sizes cover take one round
// trip; larger ones loop over further passes.
template <int YS, int TS, int BU>
__global__ void __launch_bounds__(256)
nf4_gemv_epilogue(const float* __restrict__ part_y, const float* __restrict__ part_t,
                  int splits, int tsplits, int M, int64_t N, int r, const uint16_t* __restrict__ B,
                  float scale, uint16_t* __restrict__ Y, float* __restrict__ T_out) {
  constexpr int kOut = 0x7ffffff0;
  extern __shared__ float s_dyn[];  // T [M][r] floats, then the B tile [r][64] bf16
  float* s_t = s_dyn;
  uint16_t* s_b = reinterpret_cast<uint16_t*>(s_dyn + M * r);
  const int tid = threadIdx.x;
  const int64_t n0 = (int64_t)blockIdx.x * 64;
  const int64_t n = n0 + (tid & 63);
  const bool nok = n < N;
  const int mt = tid >> 6;
  const __amdgpu_buffer_rsrc_t ry = rsrc_of(part_y, (int64_t)splits * M * N * 4);
  const __amdgpu_buffer_rsrc_t rt = rsrc_of(part_t, (int64_t)tsplits * M * r * 4);
  const __amdgpu_buffer_rsrc_t rb = rsrc_of(B, (int64_t)r * N * 2);
  // offsets in 32 bits (each range is capped below 2^31 bytes), unsigned so
  // that an unused one may wrap; an invalid load reads past the range
  const uint32_t Nu = (uint32_t)N, Mu = (uint32_t)M, ru = (uint32_t)r;
  const uint32_t nu = (uint32_t)n;
  auto ld_y = [&](int s, int m) {
    const bool ok = nok && m < M && s < splits;
    const uint32_t off = (((uint32_t)s * Mu + (uint32_t)m) * Nu + nu) * 4u;
    return __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(ry, ok ? (int)off : kOut, 0, 0));
  };
  auto ld_t = [&](int s, int e) {
    const bool ok = e < M * r && s < tsplits;
    const uint32_t off = ((uint32_t)s * Mu * ru + (uint32_t)e) * 4u;
    return __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(rt, ok ? (int)off : kOut, 0, 0));
  };
  auto ld_b = [&](int u) {  // unit u: row u / 8, columns n0 + 8 (u % 8) ..
    const bool ok = u < 8 * r;
    const uint32_t off = (((uint32_t)u >> 3) * Nu + (uint32_t)n0 + (uint32_t)(u & 7) * 8u) * 2u;
    return __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, ok ? (int)off : kOut, 0, 0));
  };
  // first pass of everything
  float py[4][YS];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int u = 0; u < YS; ++u) py[i][u] = ld_y(u, mt + 4 * i);
  u32x4 bv[BU];
#pragma unroll
  for (int q = 0; q < BU; ++q) bv[q] = ld_b(tid + 256 * q);
  float pt[TS];
#pragma unroll
  for (int u = 0; u < TS; ++u) pt[u] = ld_t(u, tid);
  float tv = 0.0f;  // first pass of T for element tid
#pragma unroll
  for (int u = 0; u < TS; ++u) tv += pt[u];

  float y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    y[i] = 0.0f;
#pragma unroll
    for (int u = 0; u < YS; ++u) y[i] += py[i][u];
  }
  for (int s0 = YS; s0 < splits; s0 += YS) {  // more splits than one pass
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int u = 0; u < YS; ++u) py[i][u] = ld_y(s0 + u, mt + 4 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int u = 0; u < YS; ++u) y[i] += py[i][u];
  }
#pragma unroll
  for (int q = 0; q < BU; ++q) {
    const int u = tid + 256 * q;
    if (u < 8 * r) *reinterpret_cast<u32x4*>(&s_b[u * 8]) = bv[q];
  }
  for (int u = tid + 256 * BU; u < 8 * r; u += 256)  // a B tile larger than one pass
    *reinterpret_cast<u32x4*>(&s_b[u * 8]) = ld_b(u);
  for (int e = tid; e < M * r; e += 256) {
    float v = tv;
    if (e != tid) {
#pragma unroll
      for (int u = 0; u < TS; ++u) pt[u] = ld_t(u, e);
      v = 0.0f;
#pragma unroll
      for (int u = 0; u < TS; ++u) v += pt[u];
    }
    for (int s0 = TS; s0 < tsplits; s0 += TS) {  // more chunks than one pass
#pragma unroll
      for (int u = 0; u < TS; ++u) pt[u] = ld_t(s0 + u, e);
#pragma unroll
      for (int u = 0; u < TS; ++u) v += pt[u];
    }
    s_t[e] = v;
    if (T_out && blockIdx.x == 0) T_out[e] = v;
  }
  __syncthreads();
  if (!nok) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = mt + 4 * i;
    if (m < M) {
      float l = 0.0f;
      for (int j = 0; j < r; ++j) l += s_t[m * r + j] * bf16_to_f32(s_b[j * 64 + (tid & 63)]);
      const float v = y[i] + scale * l;
      Y[(int64_t)m * N + n] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xffffu);
    }
  }
}

template <int YS, int TS>
void launch_epilogue_bu(int bu, dim3 grid, size_t lds, hipStream_t stream, const float* part_y,
                        const float* part_t, int splits, int tsplits, int M, int64_t N, int r,
                        const uint16_t* B, float scale, uint16_t* Y, float* T_out) {
  if (bu <= 1)
    hipLaunchKernelGGL((nf4_gemv_epilogue<YS, TS, 1>), grid, dim3(256), lds, stream, part_y,
                       part_t, splits, tsplits, M, N, r, B, scale, Y, T_out);
  else if (bu <= 2)
    hipLaunchKernelGGL((nf4_gemv_epilogue<YS, TS, 2>), grid, dim3(256), lds, stream, part_y,
                       part_t, splits, tsplits, M, N, r, B, scale, Y, T_out);
  else
    hipLaunchKernelGGL((nf4_gemv_epilogue<YS, TS, 8>), grid, dim3(256), lds, stream, part_y,
                       part_t, splits, tsplits, M, N, r, B, scale, Y, T_out);
}

// Pass sizes: the smallest of the instantiated ones that covers the shape.
void launch_epilogue(dim3 grid, size_t lds, hipStream_t stream, const float* part_y,
                     const float* part_t, int splits, int tsplits, int M, int64_t N, int r,
                     const uint16_t* B, float scale, uint16_t* Y, float* T_out) {
  const int bu = (8 * r + 255) / 256;
  if (splits <= 4 && tsplits <= 16)
    launch_epilogue_bu<4, 16>(bu, grid, lds, stream, part_y, part_t, splits, tsplits, M, N, r, B,
                              scale, Y, T_out);
  else
    launch_epilogue_bu<8, 32>(bu, grid, lds, stream, part_y, part_t, splits, tsplits, M, N, r, B,
                              scale, Y, T_out);
}

// k per GEMV workgroup: 8 packets columns of 128 (two per lane)
constexpr int kIters = 8;

}  // namespace

int64_t gemv_splits(int64_t M, int64_t K) {
  (void)M;
  const int64_t kc = (int64_t)kIters * kChunk;
  return (K + kc - 1) / kc;
}

int64_t gemv_partial_elems(int64_t M, int64_t N, int64_t K, int r) {
  if (M > kGemvMaxM) return 0;
  return gemv_splits(M, K) * M * N + (K + kTK - 1) / kTK * M * r;
}

size_t ws_offset_part(int64_t M, int64_t N, int64_t K, int r);

hipError_t launch_fwd_gemv(const uint16_t* X, Nf4Weight W, const uint16_t* A, const uint16_t* B,
                           int M, int64_t N, int64_t K, int r, float scale, uint16_t* Y,
                           float* T_out, void* ws_, hipStream_t stream, hipEvent_t ev0,
                           hipEvent_t ev1) {
  char* ws = reinterpret_cast<char*>(ws_);
  const int splits = (int)gemv_splits(M, K);
  float* part_y = reinterpret_cast<float*>(ws + ws_offset_part(M, N, K, r));
  float* part_t = part_y + (int64_t)splits * M * N;
  GemvArgs a{X, W.codes, W.absmax_q, W.absmax_s2, A, M, r, N, K,
             (int)((N + kRowsPerBlock - 1) / kRowsPerBlock), splits,
             (int)((K + kTK - 1) / kTK), (r + kTCols - 1) / kTCols, part_y, part_t};
  dim3 grid((unsigned)(a.ntiles * splits + a.tchunks * a.tblocks));
  hipError_t e = record_if(ev0, stream);
  if (e != hipSuccess) return e;
  if (W.absmax_q)
    hipLaunchKernelGGL((nf4_gemv_main<kIters, true>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((nf4_gemv_main<kIters, false>), grid, dim3(kThreads), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = record_if(ev1, stream);
  if (e != hipSuccess) return e;
  const size_t lds = (size_t)M * r * sizeof(float) + (size_t)r * 64 * sizeof(uint16_t);
  launch_epilogue(dim3((unsigned)((N + 63) / 64)), lds, stream, part_y, part_t, splits, a.tchunks,
                  M, N, r, B, scale, Y, T_out);
  return hipGetLastError();
}

}  // namespace qlora
