// Small-M forward (M <= 16): the decode-shaped product, bound by HBM.
//
//   Y = X bf16(W')^T + s (X A) B          (ozercemkelahmet.com "QLoRA",
//                                          How it works, Step 5)
//
// Two launches per call; Y is written once, by the second.
//
// 1. nf4_lowrank_kernel: partials of T = X A, one workgroup per 256-wide k
//    chunk and 16 adapter columns, the adapter's columns loaded straight into
//    MFMA operands. A few dozen workgroups; they read A and X once.
// 2. nf4_gemv_kernel: one workgroup per 16 weight rows over the whole K, so
//    that no partial of Y leaves the workgroup. Wave w of the eight owns
//    k [512 w, 512 w + 512) of each 4096-wide pass, in two steps of 256;
//    lane (c, g) owns weight row c and, in each step, the 64-block at 64 g.
//    Before any arithmetic a lane issues its code bytes (two 16-byte loads
//    per block), the blocks' 8-bit and second-level constants, and the
//    wave's slice of the token rows, which the wave alone
//    stages in its own LDS rows (no workgroup barrier before the products);
//    the adapter term's inputs (T's partials, the 16 columns of B) are
//    issued with them. Each block's 16 possible weights bf16(fl(L[q] c'))
//    are formed once (one table per 64 codes) and every code selects its two
//    bytes with v_perm_b32, straight into the B operand of
//    v_mfma_f32_16x16x32_bf16, the tokens (rows >= M zero) forming the A
//    operand. The selection leaves the eight weights of a code word in the
//    order 0, 2, 4, 6, 1, 3, 5, 7, and the token rows are staged in the same
//    order, so each MFMA sums the same products. After the passes each wave
//    adds s T B over its eighth of the ranks to its accumulators, and the
//    eight waves are summed through LDS in a fixed order. Deterministic.
#include "common.h"
#include "kernels.h"

#include <algorithm>
#include <atomic>

namespace qlora {

namespace {

constexpr int kOut = 0x7ffffff0;     // an offset past every range: the load returns 0
constexpr int kThreads = 512;        // eight waves
constexpr int kWaves = kThreads / 64;
constexpr int kRows = 16;            // weight rows per GEMV workgroup
constexpr int kStepK = 256;          // k per step of a wave: 4 lane groups x one block
constexpr int kSteps = 2;            // steps per wave and pass
constexpr int kWaveK = kSteps * kStepK;           // 512 k per wave and pass
constexpr int kPassK = kWaves * kWaveK;           // 4096 k per pass
constexpr int kXPitch = kWaveK * 2 + 16;          // LDS bytes per staged token row of a wave
constexpr int kTU = 16;              // T partials per element issued ahead of the passes
constexpr int kShortRank = 64;       // ranks whose T and B tile have LDS of their own
// adapter workgroups
constexpr int kTK = kWaves * 32;     // k per adapter workgroup (32 per wave)
constexpr int kTCols = 16;           // adapter columns per adapter workgroup
constexpr int kMaxRank = 256;  // the largest rank the linear calls accept

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* base, int64_t bytes) {
  if (bytes > 0x7ffffff0LL) bytes = 0x7ffffff0LL;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

struct LowrankArgs {
  const uint16_t* X;
  const uint16_t* A;
  int M, r;
  int64_t K;
  int tblocks;     // 16-column groups of the adapter
  float* part_t;   // [tchunks][M][r]
};

// Partial of T = X A over one kTK-wide k chunk for adapter columns
// [16 t, 16 t + 16): wave w takes the 32 k at 32 w of the chunk in one
// v_mfma_f32_16x16x32_bf16, the tokens (rows >= M zero) as the A operand and
// eight 16-bit loads of one adapter column as the B operand (no LDS
// staging: one load round trip), and the eight waves are summed through LDS
// in a fixed order.
__global__ void __launch_bounds__(kThreads) nf4_lowrank_kernel(LowrankArgs a) {
  __shared__ floatx4 s_red[kWaves][64];
  const int chunk = blockIdx.x / a.tblocks, t = blockIdx.x % a.tblocks;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, g = lane >> 4;
  const int64_t k0 = (int64_t)chunk * kTK + wave * 32 + 8 * g;  // this lane's 8 k
  const int j = t * kTCols + col;
  const __amdgpu_buffer_rsrc_t ra = rsrc_of(a.A, a.K * a.r * 2);
  const __amdgpu_buffer_rsrc_t rx = rsrc_of(a.X, (int64_t)a.M * a.K * 2);
  const u32x4 xf = __builtin_bit_cast(
      u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                 rx, (col < a.M && k0 < a.K) ? (int)(((int64_t)col * a.K + k0) * 2) : kOut, 0, 0));
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const bool ok = k0 + e < a.K && j < a.r;
    h[e] = __builtin_amdgcn_raw_buffer_load_b16(ra, ok ? (int)(((k0 + e) * a.r + j) * 2) : kOut, 0, 0);
  }
  u32x4 wb;
#pragma unroll
  for (int e = 0; e < 4; ++e) wb[e] = (h[2 * e] & 0xffffu) | (h[2 * e + 1] << 16);
  const floatx4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
  s_red[wave][lane] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xf), as_bf16x8(wb), zero, 0, 0, 0);
  __syncthreads();
  if (wave == 0 && j < a.r) {
    floatx4 tt = s_red[0][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      const floatx4 u = s_red[w][lane];
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

struct GemvArgs {
  const uint16_t* X;
  const uint8_t* codes;
  const uint8_t* absmax_q;
  const float* absmax_s2;
  const uint16_t* B;
  int M, r;
  int64_t N, K;
  int tchunks;     // partials of T
  const float* part_t;
  float scale;
  uint16_t* Y;
  float* T_out;    // optional
  Codebook cb;     // levels and constant code of the store type
};

// kMX: the largest M the instantiation serves (4 or 16: the token rows a
// wave stages per pass). kDQ false: the store has no 8-bit codes and
// absmax_s2 holds one float32 constant per block.
template <int kMX, bool kDQ>
__global__ void __launch_bounds__(kThreads) nf4_gemv_kernel(GemvArgs a) {
#pragma clang fp contract(off)
  // each wave's token rows of one pass, [M][kWaveK] at kXPitch bytes a row,
  // and a row of zeros ((M + 1) * kXPitch bytes a wave); after the passes:
  // T [M][r] float32, then the B tile [r][16] bf16
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  __shared__ floatx4 s_red[kWaves][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, g = lane >> 4;
  const int M = a.M, r = a.r;
  const int64_t K = a.K;
  const int64_t n0 = (int64_t)blockIdx.x * kRows;
  const int64_t n = n0 + col;  // < N: N is a multiple of 64
  const int mr = M * r;
  // the wave's LDS rows: M token rows, then one row of zeros that the lanes
  // of tokens >= M read, so that no MFMA operand needs a branch
  uint8_t* xw = dyn + wave * ((M + 1) * kXPitch);
  const uint8_t* xrow = xw + (col < M ? col : M) * kXPitch;
  *reinterpret_cast<u32x4*>(xw + M * kXPitch + lane * 16) = u32x4{0u, 0u, 0u, 0u};

  const __amdgpu_buffer_rsrc_t rc = rsrc_of(a.codes, a.N * K / 2);
  const __amdgpu_buffer_rsrc_t rq = rsrc_of(a.absmax_q, kDQ ? a.N * K / kBlock : 0);
  const __amdgpu_buffer_rsrc_t rs =
      rsrc_of(a.absmax_s2, kDQ ? (a.N * K / kBlock + kGroup - 1) / kGroup * 4 : a.N * K / kBlock * 4);
  const __amdgpu_buffer_rsrc_t rx = rsrc_of(a.X, (int64_t)M * K * 2);
  const __amdgpu_buffer_rsrc_t rt = rsrc_of(a.part_t, (int64_t)a.tchunks * mr * 4);
  const __amdgpu_buffer_rsrc_t rb = rsrc_of(a.B, (int64_t)r * a.N * 2);

  floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  // adapter-term inputs, issued with the first pass by the waves that hold
  // them: the first kTU partials of T element tid, and unit tid of the B
  // tile (row tid / 2, 8 columns)
  float tp[kTU];
#pragma unroll
  for (int u = 0; u < kTU; ++u) tp[u] = 0.0f;
  u32x4 bv = u32x4{0u, 0u, 0u, 0u};
  const int npass = (int)((K + kPassK - 1) / kPassK);
  for (int pass = 0; pass < npass; ++pass) {
    // this wave's k range of the pass
    const int64_t kw = (int64_t)pass * kPassK + (int64_t)wave * kWaveK;
    // token rows: lane l loads k = kw + 8 l .. + 8 of each row < M (an
    // invalid load returns 0)
    u32x4 xr[kMX];
    const bool kx = kw + 8 * lane < K;
#pragma unroll
    for (int m = 0; m < kMX; ++m) {
      xr[m] = u32x4{0u, 0u, 0u, 0u};
      if (m < M)  // uniform
        xr[m] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                       rx, kx ? (int)(((int64_t)m * K + kw + 8 * lane) * 2) : kOut, 0, 0));
    }
    // codes: step s, lane group g holds the 64-block at kw + 256 s + 64 g of
    // row n (32 bytes), with its 8-bit and second-level constants
    u32x4 c[kSteps][2];
    uint32_t q8[kSteps];
    float s2[kSteps];
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const int64_t k = kw + st * kStepK + 64 * g;
      const bool ok = k < K;
      const int64_t e = n * K + k;
#pragma unroll
      for (int h = 0; h < 2; ++h)
        c[st][h] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, ok ? (int)(e / 2 + 16 * h) : kOut, 0, 0));
      const int64_t b = e / kBlock;
      if constexpr (kDQ) {
        q8[st] = __builtin_amdgcn_raw_buffer_load_b8(rq, ok ? (int)b : kOut, 0, 0);
        s2[st] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rs, ok ? (int)((b / kGroup) * 4) : kOut, 0, 0));
      } else {
        q8[st] = 255u;
        s2[st] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(rs, ok ? (int)(b * 4) : kOut, 0, 0));
      }
    }
    if (pass == 0) {
      if (wave * 64 < mr) {  // uniform
#pragma unroll
        for (int u = 0; u < kTU; ++u)
          tp[u] = __builtin_bit_cast(
              float, __builtin_amdgcn_raw_buffer_load_b32(
                         rt, (tid < mr && u < a.tchunks) ? (int)(((int64_t)u * mr + tid) * 4) : kOut,
                         0, 0));
      }
      if (wave * 64 < 2 * r)  // uniform
        bv = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                       rb, tid < 2 * r ? (int)((((int64_t)(tid >> 1)) * a.N + n0 + 8 * (tid & 1)) * 2) : kOut,
                       0, 0));
    }
    // the wave's token rows into its LDS rows, in the element order of the
    // dequantized weights; LDS accesses of one wave complete in order, so
    // the reads below see these writes (and the previous pass's reads came
    // before them)
    asm volatile("" ::: "memory");
#pragma unroll
    for (int m = 0; m < kMX; ++m)
      if (m < M) *reinterpret_cast<u32x4*>(xw + m * kXPitch + lane * 16) = x_order_oddeven(xr[m]);
    asm volatile("" ::: "memory");

#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      const float cs = !kDQ ? s2[st]
                       : a.cb.dq_fp8 ? block_scale_fp8(q8[st], s2[st]) : block_scale(q8[st], s2[st]);
      const PermTable pt = perm_table(cs, a.cb.lv);  // lookups by v_perm: no LDS round trips
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        // MFMA t takes this lane's codes 8 t .. 8 t + 7 and the same k of the
        // token rows, both in the odd-even element order
        const u32x4 xv = *reinterpret_cast<const u32x4*>(xrow + (st * kStepK + 64 * g + 8 * t) * 2);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(xv), as_bf16x8(dequant_word_perm_oddeven(c[st][t >> 2][t & 3], pt)), acc, 0, 0,
            0);
      }
    }
    asm volatile("" ::: "memory");
  }
  // The adapter term: T (the sum of its partials in chunk order) and the B
  // tile go to LDS, after the token rows for ranks up to kShortRank (written
  // as soon as a wave is done), else in the token rows' LDS once every wave
  // is done with it; each wave then adds s T B over its eighth of the ranks.
  const bool short_rank = r <= kShortRank;  // uniform
  uint8_t* tb = short_rank ? dyn + kWaves * (M + 1) * kXPitch : dyn;
  if (!short_rank) __syncthreads();
  float* s_t = reinterpret_cast<float*>(tb);
  uint16_t* s_b = reinterpret_cast<uint16_t*>(tb + ((mr * 4 + 15) & ~15));
  if (tid < mr) {
    float v = 0.0f;
#pragma unroll
    for (int u = 0; u < kTU; ++u) v += tp[u];  // partials past tchunks read 0
    for (int u = kTU; u < a.tchunks; ++u)
      v += a.part_t[(int64_t)u * mr + tid];
    s_t[tid] = v;
    if (a.T_out && blockIdx.x == 0) a.T_out[tid] = v;
  }
  for (int e = tid + kThreads; e < mr; e += kThreads) {  // more elements than threads
    float v = 0.0f;
    for (int u = 0; u < a.tchunks; ++u) v += a.part_t[(int64_t)u * mr + e];
    s_t[e] = v;
    if (a.T_out && blockIdx.x == 0) a.T_out[e] = v;
  }
  if (tid < 2 * r) *reinterpret_cast<u32x4*>(s_b + tid * 8) = bv;

  // D[i][j] of the MFMA: this lane holds tokens i = 4 g + v of weight row
  // j = col. l = sum over a range of ranks of T[i][j'] B[j'][col].
  auto lora = [&](int jb, int je, float (&l)[4]) {
    for (int j = jb; j < je; ++j) {
      const float bj = bf16_to_f32(s_b[j * kRows + col]);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 4 * g + v;
        if (m < M) l[v] += s_t[m * r + j] * bj;
      }
    }
  };
  __syncthreads();
  {
    float l[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    const int r8 = (r + kWaves - 1) / kWaves;
    lora(wave * r8, min(r, wave * r8 + r8), l);
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] += a.scale * l[v];
  }
  s_red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    floatx4 y = s_red[0][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      const floatx4 u = s_red[w][lane];
#pragma unroll
      for (int v = 0; v < 4; ++v) y[v] += u[v];
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * g + v;
      if (m < M) a.Y[(int64_t)m * a.N + n] = (uint16_t)(pack_bf16x2(y[v], 0.0f) & 0xffffu);
    }
  }
}

int64_t tchunks_of(int64_t K) { return (K + kTK - 1) / kTK; }

size_t gemv_lds_bytes(int M, int r) {
  const size_t x = (size_t)kWaves * (M + 1) * kXPitch;
  const size_t tb = (size_t)((M * r * 4 + 15) & ~15) + (size_t)r * kRows * 2;
  return r <= kShortRank ? x + tb : std::max(x, tb);
}

// The dynamic LDS limit is raised once per device and instantiation, to the
// largest size any call asks for (sixteen staged token rows).
template <int kMX, bool kDQ>
hipError_t launch_gemv_kernel(const GemvArgs& a, size_t lds, hipStream_t stream) {
  auto kern = nf4_gemv_kernel<kMX, kDQ>;
  static std::atomic<uint64_t> raised{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (!(raised.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)std::max(gemv_lds_bytes(kMX, kShortRank), gemv_lds_bytes(kMX, kMaxRank)));
    if (e != hipSuccess) return e;
    raised.fetch_or(bit, std::memory_order_acq_rel);
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)(a.N / kRows)), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace

int64_t gemv_partial_elems(int64_t M, int64_t N, int64_t K, int r) {
  (void)N;
  if (M > kGemvMaxM) return 0;
  return tchunks_of(K) * M * r;
}

size_t ws_offset_part(int64_t M, int64_t N, int64_t K, int r);

hipError_t launch_fwd_gemv(const uint16_t* X, Nf4Weight W, const uint16_t* A, const uint16_t* B,
                           int M, int64_t N, int64_t K, int r, float scale, uint16_t* Y,
                           float* T_out, void* ws_, hipStream_t stream, hipEvent_t ev0,
                           hipEvent_t ev1) {
  char* ws = reinterpret_cast<char*>(ws_);
  float* part_t = reinterpret_cast<float*>(ws + ws_offset_part(M, N, K, r));
  const int tchunks = (int)tchunks_of(K);
  const int tblocks = (r + kTCols - 1) / kTCols;
  LowrankArgs la{X, A, M, r, K, tblocks, part_t};
  hipLaunchKernelGGL(nf4_lowrank_kernel, dim3((unsigned)(tchunks * tblocks)), dim3(kThreads), 0,
                     stream, la);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  GemvArgs a{X, W.codes, W.absmax_q, W.absmax_s2, B, M, r, N, K, tchunks, part_t, scale, Y,
             T_out, codebook_of(W)};
  const size_t lds = gemv_lds_bytes(M, r);
  e = record_if(ev0, stream);
  if (e != hipSuccess) return e;
  if (M <= 4)
    e = W.absmax_q ? launch_gemv_kernel<4, true>(a, lds, stream)
                   : launch_gemv_kernel<4, false>(a, lds, stream);
  else
    e = W.absmax_q ? launch_gemv_kernel<16, true>(a, lds, stream)
                   : launch_gemv_kernel<16, false>(a, lds, stream);
  if (e != hipSuccess) return e;
  return record_if(ev1, stream);
}

}  // namespace qlora
