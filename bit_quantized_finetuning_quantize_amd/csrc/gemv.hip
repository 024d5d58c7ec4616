// Small-M forward (M <= 16): the decode-shaped product, bound by HBM.
//
//   Y = X bf16(W')^T + s (X A) B          (ozercemkelahmet.com "QLoRA",
//                                          How it works, Step 5)
//
// One launch per call, two kinds of workgroup; Y is written once.
//
// 1. Producers (the first 8 * tchunks * tblocks workgroups): partials of
//    T = X A, one workgroup per 256-wide k chunk, 16 adapter columns and XCD,
//    the adapter's columns loaded straight into MFMA operands. Each writes
//    its partial to its XCD's copy and then a flag holding the call's tag.
// 2. Consumers: one workgroup per 16 weight rows over the whole K, so
//    that no partial of Y leaves the workgroup. Wave w of the eight owns
//    k [512 w, 512 w + 512) of each 4096-wide pass, in two steps of 256;
//    lane (c, g) owns weight row c and, in each step, the 64-block at 64 g.
//    Before any arithmetic a lane issues its code bytes (two 16-byte loads
//    per block), the blocks' 8-bit and second-level constants, and the
//    wave's slice of the token rows, which the wave alone
//    stages in its own LDS rows (no workgroup barrier before the products);
//    the 16 columns of B are issued with them. Each block's 16 possible
//    weights bf16(fl(L[q] c')) are formed once (one table per 64 codes) and
//    every code selects its two bytes with v_perm_b32, straight into the B
//    operand of v_mfma_f32_16x16x32_bf16, the tokens (rows >= M zero)
//    forming the A operand. The selection leaves the eight weights of a code
//    word in the order 0, 2, 4, 6, 1, 3, 5, 7, and the token rows are staged
//    in the same order, so each MFMA sums the same products. Only after the
//    passes does a consumer need T: it waits for the flags of its XCD's
//    producers, sums the partials in chunk order, adds s T B over its eighth
//    of the ranks to each wave's accumulators, and the eight waves are summed
//    through LDS in a fixed order. Deterministic.
//
// The handover. A launch's workgroups are dealt to the 8 XCDs in turn, so
// producer i runs on XCD i mod 8 and each XCD has a producer for every
// tile; the partials and flags stay in that XCD's L2, which all of its CUs
// share, and never wait for HBM. Producers have the lowest workgroup ids:
// each is placed before any consumer of its XCD and never waits on one,
// and their work is hidden behind the consumers' weight stream, where a
// launch of its own cost a whole launch gap. A flag carries a tag unique to
// the dispatch (the packet's index in its queue, mixed with the queue's
// address), so the workspace needs no clearing between calls and its
// contents on entry do not matter. A producer waits for the L2 to take its
// partials before it stores the flag; a consumer polls the flag with atomic
// additions of zero, which the L2 performs (a plain load could be served by
// the CU's L1 from a line read before the flag was set), and reads the
// partials only then, lines that no wave of its CU has read before in this
// launch. The XCD is read from the hardware, so a workgroup uses its own
// XCD's copy wherever it is placed; if a consumer has not seen every flag
// within a bounded time (a placement that left a tile without a producer on
// its XCD would do that), it forms the partials itself, chunk by chunk in
// the same order and arithmetic, so the result is the same bit for bit
// either way.
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
// Token rows a wave stages at once: both steps of a pass for M <= 4; one
// step at a time for more tokens, which halves the LDS of a workgroup (to
// 78 KiB at 16 tokens), so that a producer fits on a CU beside a consumer
// and all workgroups of a 4096-row call are placed at once.
constexpr int staged_steps(int M) { return M > 4 ? 1 : kSteps; }
constexpr int x_pitch(int M) { return staged_steps(M) * kStepK * 2 + 16; }  // LDS bytes a row
constexpr int kTU = 16;              // T partials a consumer thread loads at once
constexpr int kShortRank = 64;       // ranks whose T and B tile have LDS of their own
// adapter workgroups
constexpr int kTK = kWaves * 32;     // k per adapter workgroup (32 per wave)
constexpr int kTCols = 16;           // adapter columns per adapter workgroup
constexpr int kMaxRank = 256;  // the largest rank the linear calls accept
// How long a consumer waits for the producers' flags before forming T
// itself, in microseconds (the real-time counter runs at 100 MHz); by
// default far beyond the few microseconds the producers take. 0 launches no
// producers: every consumer forms T.
std::atomic<int64_t> g_wait_us{200};
constexpr int kSpinPolls = 1 << 16;  // a bound on polls as well
constexpr int kXcds = 8;       // XCDs of the device, each with its own L2

// The dispatch packet's index in its queue (a hardware-provided value).
extern "C" __device__ uint64_t qlora_dispatch_index() __asm("llvm.amdgcn.dispatch.id");

// The XCD this wave runs on (its L2 is shared by that XCD's CUs only).
__device__ __forceinline__ int xcd_id() {
  unsigned v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return (int)(v & (kXcds - 1));
}

// Flags sit 128 bytes apart, one to an L2 line.
constexpr int kFlagStride = 16;  // u64 elements

// A tag unique to this dispatch within the process: dispatch indices count
// up per queue, and queues differ in address bits 12-39, so the value
// repeats only after 2^36 dispatches on one queue.
__device__ __forceinline__ uint64_t call_tag() {
  const uint64_t q = (uint64_t)(uintptr_t)__builtin_amdgcn_queue_ptr();
  return qlora_dispatch_index() ^ (q << 24);
}

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
  const uint16_t* B;
  int M, r;
  int64_t N, K;
  int tchunks;     // k chunks of T's partials
  int tblocks;     // 16-column groups of the adapter
  int nprod;       // partial tiles of T launched: tchunks * tblocks (kXcds producers
                   // each), or 0 (the consumers form T)
  uint64_t spin_ticks;  // how long a consumer polls, in real-time counter ticks
  float* part_t;   // [kXcds][tchunks][M][r]
  uint64_t* flags; // [kXcds][nprod]
  float scale;
  uint16_t* Y;
  float* T_out;    // optional
  Codebook cb;     // levels and constant code of the store type
};

// Partial of T = X A over the kTK-wide k chunk `chunk` for adapter columns
// [16 t, 16 t + 16): wave w takes the 32 k at 32 w of the chunk in one
// v_mfma_f32_16x16x32_bf16, the tokens (rows >= M zero) as the A operand and
// eight 16-bit loads of one adapter column as the B operand (no LDS
// staging: one load round trip), and the eight waves are summed through LDS
// in a fixed order. Called by every thread of the workgroup; returns, in
// wave 0, tokens 4 g + v (v < 4) of adapter column 16 t + (lane & 15).
__device__ __forceinline__ floatx4 lowrank_partial(const GemvArgs& a, int chunk, int t,
                                                   floatx4 (*s_red)[64]) {
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
  floatx4 tt = zero;
  if (wave == 0) {
    tt = s_red[0][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      const floatx4 u = s_red[w][lane];
#pragma unroll
      for (int v = 0; v < 4; ++v) tt[v] += u[v];
    }
  }
  __syncthreads();  // s_red is free again
  return tt;
}

// kMX: the largest M the instantiation serves (4 or 16: the token rows a
// wave stages per pass). kDQ false: the store has no 8-bit codes and
// absmax_s2 holds one float32 constant per block.
template <int kMX, bool kDQ>
__global__ void __launch_bounds__(kThreads) nf4_gemv_kernel(GemvArgs a) {
#pragma clang fp contract(off)
  // each wave's token rows of one pass (or step), [M][kStaged * kStepK] at
  // kPitch bytes a row, and a row of zeros ((M + 1) * kPitch bytes a wave);
  // after the passes: T [M][r] float32, then the B tile [r][16] bf16
  constexpr int kStaged = staged_steps(kMX);
  constexpr int kPitch = x_pitch(kMX);
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  __shared__ floatx4 s_red[kWaves][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, g = lane >> 4;
  const int M = a.M, r = a.r;
  const int64_t K = a.K;
  const uint64_t tag = call_tag();
  const int x = xcd_id();
  const int nprod_all = kXcds * a.nprod;
  if ((int)blockIdx.x < nprod_all) {  // a producer (uniform)
    const int p = blockIdx.x / kXcds;  // its tile; XCD x's copy of it
    const int chunk = p / a.tblocks, t = p % a.tblocks;
    const floatx4 tt = lowrank_partial(a, chunk, t, s_red);
    if (wave == 0) {
      const int j = t * kTCols + col;
      float* part = a.part_t + (int64_t)x * a.tchunks * M * r;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 4 * g + v;
        if (m < M && j < r)
          __hip_atomic_store(part + ((int64_t)chunk * M + m) * r + j, tt[v], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      // every store of the wave acknowledged by the L2 before the flag
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      if (lane == 0)
        __hip_atomic_store(a.flags + ((int64_t)x * a.nprod + p) * kFlagStride, tag,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    return;
  }
  const int64_t n0 = (int64_t)(blockIdx.x - nprod_all) * kRows;
  const int64_t n = n0 + col;  // < N: N is a multiple of 64
  const int mr = M * r;
  // the wave's LDS rows: M token rows, then one row of zeros that the lanes
  // of tokens >= M read, so that no MFMA operand needs a branch
  uint8_t* xw = dyn + wave * ((M + 1) * kPitch);
  const uint8_t* xrow = xw + (col < M ? col : M) * kPitch;
  if (lane * 16 < kStaged * kStepK * 2)
    *reinterpret_cast<u32x4*>(xw + M * kPitch + lane * 16) = u32x4{0u, 0u, 0u, 0u};

  const __amdgpu_buffer_rsrc_t rc = rsrc_of(a.codes, a.N * K / 2);
  const __amdgpu_buffer_rsrc_t rq = rsrc_of(a.absmax_q, kDQ ? a.N * K / kBlock : 0);
  const __amdgpu_buffer_rsrc_t rs =
      rsrc_of(a.absmax_s2, kDQ ? (a.N * K / kBlock + kGroup - 1) / kGroup * 4 : a.N * K / kBlock * 4);
  const __amdgpu_buffer_rsrc_t rx = rsrc_of(a.X, (int64_t)M * K * 2);
  const __amdgpu_buffer_rsrc_t rb = rsrc_of(a.B, (int64_t)r * a.N * 2);

  floatx4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  // the B tile, issued with the first pass by the waves that hold it: unit
  // tid is row tid / 2, 8 columns
  u32x4 bv = u32x4{0u, 0u, 0u, 0u};
  const int npass = (int)((K + kPassK - 1) / kPassK);
  for (int pass = 0; pass < npass; ++pass) {
    // this wave's k range of the pass
    const int64_t kw = (int64_t)pass * kPassK + (int64_t)wave * kWaveK;
    // token rows (an invalid load returns 0). All of a pass at once for
    // kStaged = 2: lane l loads k = kw + 8 l .. + 8 of each row < M. One step
    // at a time otherwise: for step s, lane l loads k = kw + 256 s + 8 (l % 32)
    // .. + 8 of rows 2 i + l / 32, i < kMX / 2 (half the registers), the
    // second step's loads issued once the first step's rows are staged.
    constexpr int kXR = kStaged == kSteps ? kMX : kMX / 2;
    u32x4 xr[kXR];
    auto load_x = [&](int st) {
#pragma unroll
      for (int i = 0; i < kXR; ++i) {
        const int m = kStaged == kSteps ? i : 2 * i + (lane >> 5);
        const int64_t k = kStaged == kSteps ? kw + 8 * lane : kw + st * kStepK + 8 * (lane & 31);
        xr[i] = u32x4{0u, 0u, 0u, 0u};
        if ((kStaged == kSteps ? i : 2 * i) < M)  // uniform
          xr[i] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                         rx, (m < M && k < K) ? (int)(((int64_t)m * K + k) * 2) : kOut, 0, 0));
      }
    };
    load_x(0);
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
      if (wave * 64 < 2 * r)  // uniform
        bv = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                       rb, tid < 2 * r ? (int)((((int64_t)(tid >> 1)) * a.N + n0 + 8 * (tid & 1)) * 2) : kOut,
                       0, 0));
    }
#pragma unroll
    for (int st = 0; st < kSteps; ++st) {
      // the wave's token rows into its LDS rows (a pass, or this step, as
      // loaded above), in the element order of the dequantized weights; LDS
      // accesses of one wave complete in order, so the reads below see these
      // writes, and the reads of the step or pass before came before them
      if (st % kStaged == 0) {
        asm volatile("" ::: "memory");
#pragma unroll
        for (int i = 0; i < kXR; ++i) {
          const int m = kStaged == kSteps ? i : 2 * i + (lane >> 5);
          const int off = kStaged == kSteps ? lane * 16 : (lane & 31) * 16;
          if (m < M) *reinterpret_cast<u32x4*>(xw + m * kPitch + off) = x_order_oddeven(xr[i]);
        }
        asm volatile("" ::: "memory");
        if (kStaged != kSteps && st + 1 < kSteps) load_x(st + 1);
      }
      const float cs = !kDQ ? s2[st]
                       : a.cb.dq_fp8 ? block_scale_fp8(q8[st], s2[st]) : block_scale(q8[st], s2[st]);
      const PermTable pt = perm_table(cs, a.cb.lv);  // lookups by v_perm: no LDS round trips
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        // MFMA t takes this lane's codes 8 t .. 8 t + 7 and the same k of the
        // token rows, both in the odd-even element order
        const u32x4 xv =
            *reinterpret_cast<const u32x4*>(xrow + ((st % kStaged) * kStepK + 64 * g + 8 * t) * 2);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(xv), as_bf16x8(dequant_word_perm_oddeven(c[st][t >> 2][t & 3], pt)), acc, 0, 0,
            0);
      }
    }
    asm volatile("" ::: "memory");
  }
  // The adapter term: T (the sum of its partials in chunk order) and the B
  // tile go to LDS, after the token rows for ranks up to kShortRank, else
  // in the token rows' LDS once every wave is done with it (the barrier of
  // the wait below); each wave then adds s T B over its eighth of the ranks.
  const bool short_rank = r <= kShortRank;  // uniform
  uint8_t* tb = short_rank ? dyn + kWaves * (M + 1) * kPitch : dyn;
  float* s_t = reinterpret_cast<float*>(tb);
  uint16_t* s_b = reinterpret_cast<uint16_t*>(tb + ((mr * 4 + 15) & ~15));
  // Wait for every producer's flag of this XCD (or the time to run out).
  // The polls are atomic additions of zero, which the L2 performs: the CU's
  // L1 would serve a plain load from a line it read before the flag was
  // set. The zero comes from an argument, so that the compiler keeps the
  // addition.
  bool seen = a.nprod > 0;
  if (seen) {
    uint64_t* flags = a.flags + (int64_t)x * a.nprod * kFlagStride;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    int polls = 0;  // a second bound, in case the clock does not advance
    const uint64_t zero = (uint64_t)(a.M >> 30);
    for (int f = tid; f < a.nprod && seen; f += kThreads)
      while (__hip_atomic_fetch_add(flags + f * kFlagStride, zero, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_WORKGROUP) != tag) {
        if (__builtin_amdgcn_s_memrealtime() - t0 > a.spin_ticks || ++polls > kSpinPolls) {
          seen = false;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
  }
  if (__syncthreads_and(seen)) {
    const float* part = a.part_t + (int64_t)x * a.tchunks * mr;
    for (int e = tid; e < mr; e += kThreads) {
      float v = 0.0f;
      for (int u0 = 0; u0 < a.tchunks; u0 += kTU) {  // kTU loads in flight, then their sum
        float pv[kTU];
#pragma unroll
        for (int i = 0; i < kTU; ++i)
          pv[i] = __hip_atomic_load(part + (int64_t)min(u0 + i, a.tchunks - 1) * mr + e,
                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
        for (int i = 0; i < kTU; ++i)
          if (u0 + i < a.tchunks) v += pv[i];
      }
      s_t[e] = v;
    }
  } else {  // form the partials here, in the same order and arithmetic
    for (int e = tid; e < mr; e += kThreads) s_t[e] = 0.0f;
    for (int u = 0; u < a.tchunks; ++u)
      for (int t = 0; t < a.tblocks; ++t) {
        const floatx4 tt = lowrank_partial(a, u, t, s_red);  // barriers inside
        const int j = t * kTCols + col;
        if (wave == 0 && j < r) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int m = 4 * g + v;
            if (m < M) s_t[m * r + j] += tt[v];
          }
        }
      }
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
  if (a.T_out && (int)blockIdx.x == nprod_all)
    for (int e = tid; e < mr; e += kThreads) a.T_out[e] = s_t[e];
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
  const size_t x = (size_t)kWaves * (M + 1) * x_pitch(M);
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
  hipLaunchKernelGGL(kern, dim3((unsigned)(kXcds * a.nprod + a.N / kRows)), dim3(kThreads), lds,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

void set_gemv_wait_us(int64_t us) { g_wait_us.store(us, std::memory_order_relaxed); }

int64_t gemv_partial_elems(int64_t M, int64_t N, int64_t K, int r) {
  (void)N;
  if (M > kGemvMaxM) return 0;
  const int64_t nprod = tchunks_of(K) * ((r + kTCols - 1) / kTCols);
  // one copy of the partials and flags per XCD; the flags 128-byte aligned
  return kXcds * ((tchunks_of(K) * M * r + 31) / 32 * 32 + 2 * kFlagStride * nprod);
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
  uint64_t* flags =
      reinterpret_cast<uint64_t*>(part_t + kXcds * (((int64_t)tchunks * M * r + 31) / 32 * 32));
  const int64_t wait_us = g_wait_us.load(std::memory_order_relaxed);
  GemvArgs a{X, W.codes, W.absmax_q, W.absmax_s2, A, B, M, r, N, K, tchunks, tblocks,
             wait_us > 0 ? tchunks * tblocks : 0, (uint64_t)wait_us * 100, part_t, flags, scale,
             Y, T_out, codebook_of(W)};
  const size_t lds = gemv_lds_bytes(M, r);
  hipError_t e = record_if(ev0, stream);
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
