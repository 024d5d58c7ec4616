// Tiled bf16 MFMA contraction with warp-specialized producers.
//
//   C[p][q] = sum_c  Aop[p][c] * Bop[q][c]      (float32 accumulation)
//
// A workgroup owns a PT x QT tile of C and walks the contraction in steps of
// 64. Waves 0-3 are consumers: each holds a (PT/2) x (QT/2) accumulator and
// issues v_mfma_f32_32x32x16_bf16 on operand tiles read from LDS. Waves 4-7
// are producers: they fetch the next steps from global memory into
// registers, convert them (NF4 dequantization, transposition, float ->
// bfloat16) and write them into the other half of a double-buffered LDS
// stage, so the VALU work of dequantization overlaps the matrix cores.
//
// Operand tiles in LDS are [rows][64] bfloat16 with the contraction index
// contiguous and rows padded to 72 elements (144 bytes), so that the 32
// lanes reading one 16-byte fragment column touch distinct banks.
//
// A contraction may have two segments: steps [0, S1) come from one pair of
// loaders and steps [S1, S1 + S2) from a second pair. The forward pass uses
// the second segment for the adapter term (s T) B, the input-gradient pass
// for (s G) A^T, so the LoRA products are accumulated by the same MFMA
// tiles as the frozen-weight product.
#pragma once

#include "common.h"

namespace qlora {
namespace gemm {

constexpr int kStep = 64;                 // contraction elements per step
constexpr int kLdsStride = 72;            // bf16 elements per LDS row
constexpr int kThreads = 512;             // 4 consumer + 4 producer waves
constexpr int kProducerThreads = 256;

__device__ __forceinline__ u32x4 ld_global_16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st_lds_16(uint16_t* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}
__device__ __forceinline__ void st_lds_8(uint16_t* p, u32x2 v) {
  *reinterpret_cast<u32x2*>(p) = v;
}

// ---------------------------------------------------------------------------
// Loaders. Each has   Regs   (what one producer thread holds for one step),
//   load(step, regs)        global -> registers (guarded, zero fill),
//   store(regs, tile, lv)   registers -> LDS tile [R][72].
// `step` counts 64-wide contraction steps from the start of the segment.

// Rows of a row-major bf16 matrix with the contraction index contiguous:
// tile row i = source row row0 + i, columns c0 .. c0+63.
template <int R>
struct LoadBf16Rows {
  static constexpr int kChunks = R * 8 / kProducerThreads;  // 16-byte chunks per thread
  const uint16_t* base;
  int64_t ld;        // elements between source rows
  int64_t rows;      // valid source rows
  int64_t cols;      // valid contraction length (multiple of 8)
  int64_t row0;
  __device__ __forceinline__ void set_origin(int64_t o) { row0 = o; }
  struct Regs { u32x4 v[kChunks]; };
  __device__ __forceinline__ void load(int step, Regs& r, int t) const {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int id = t + i * kProducerThreads;
      const int row = id >> 3, ch = id & 7;
      const int64_t gr = row0 + row;
      const int64_t gc = (int64_t)step * kStep + ch * 8;
      if (gr < rows && gc < cols)
        r.v[i] = ld_global_16(base + gr * ld + gc);
      else
        r.v[i] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(const Regs& r, uint16_t* tile, const float*, int t) const {
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int id = t + i * kProducerThreads;
      const int row = id >> 3, ch = id & 7;
      st_lds_16(tile + row * kLdsStride + ch * 8, r.v[i]);
    }
  }
};

// Transposed bf16 source: tile row i = source COLUMN col0 + i, contraction
// index = source row. Each thread moves 4 source rows x 8 source columns.
template <int R>
struct LoadBf16Cols {
  static constexpr int kUnits = R * 2;                       // (4 x 8) units per tile
  static constexpr int kPer = (kUnits + kProducerThreads - 1) / kProducerThreads;
  const uint16_t* base;
  int64_t ld;        // elements between source rows
  int64_t rows;      // valid source rows (contraction length)
  int64_t cols;      // valid source columns (multiple of 8)
  int64_t col0;
  __device__ __forceinline__ void set_origin(int64_t o) { col0 = o; }
  struct Regs { u32x4 v[kPer][4]; };
  __device__ __forceinline__ void load(int step, Regs& r, int t) const {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int id = t + u * kProducerThreads;
      const int rg = id % (R / 8), cg = id / (R / 8);
      const int64_t gcol = col0 + rg * 8;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t grow = (int64_t)step * kStep + cg * 4 + e;
        if (id < kUnits && grow < rows && gcol < cols)
          r.v[u][e] = ld_global_16(base + grow * ld + gcol);
        else
          r.v[u][e] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  __device__ __forceinline__ void store(const Regs& r, uint16_t* tile, const float*, int t) const {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int id = t + u * kProducerThreads;
      if (id >= kUnits) continue;
      const int rg = id % (R / 8), cg = id / (R / 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // element e of each of the 4 source rows
        const int w = e >> 1, sh = (e & 1) * 16;
        const uint32_t a0 = (r.v[u][0][w] >> sh) & 0xffffu;
        const uint32_t a1 = (r.v[u][1][w] >> sh) & 0xffffu;
        const uint32_t a2 = (r.v[u][2][w] >> sh) & 0xffffu;
        const uint32_t a3 = (r.v[u][3][w] >> sh) & 0xffffu;
        st_lds_8(tile + (rg * 8 + e) * kLdsStride + cg * 4,
                 u32x2{a0 | (a1 << 16), a2 | (a3 << 16)});
      }
    }
  }
};

// NF4 weight rows (forward): tile row i = weight row n0 + i (output feature),
// contraction = input feature k; one step is exactly one 64-value block of a
// row. Two threads per row, 32 codes each.
template <int R>
struct LoadNf4Rows {
  static_assert(R * 2 == kProducerThreads, "two producer threads per row");
  const uint8_t* codes;
  const uint8_t* absmax_q;
  const float* absmax_s2;
  int64_t N, K, n0;
  __device__ __forceinline__ void set_origin(int64_t o) { n0 = o; }
  struct Regs { u32x4 c; uint32_t q8; float s2; };
  __device__ __forceinline__ void load(int step, Regs& r, int t) const {
    const int row = t >> 1, half = t & 1;
    const int64_t n = n0 + row;
    if (n < N) {
      const int64_t e = n * K + (int64_t)step * kStep + half * 32;
      r.c = ld_global_16(codes + e / 2);
      const int64_t b = e / kBlock;
      r.q8 = absmax_q[b];
      r.s2 = absmax_s2[b / kGroup];
    } else {
      r.c = u32x4{0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u};
      r.q8 = 0;
      r.s2 = 0.0f;
    }
  }
  __device__ __forceinline__ void store(const Regs& r, uint16_t* tile, const float* lv, int t) const {
    const int row = t >> 1, half = t & 1;
    const float cs = block_scale(r.q8, r.s2);
    uint16_t* dst = tile + row * kLdsStride + half * 32;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t c = r.c[w];
      u32x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float lo = lv[(c >> (8 * j)) & 15u] * cs;
        const float hi = lv[(c >> (8 * j + 4)) & 15u] * cs;
        o[j] = pack_bf16x2(lo, hi);
      }
      st_lds_16(dst + w * 8, o);
    }
  }
};

// NF4 weight, transposed (input gradient): tile row i = input feature
// k0 + i, contraction = output feature n. Each thread dequantizes 4 weight
// rows x 8 consecutive k (one 32-bit code word per row).
template <int R>
struct LoadNf4Cols {
  static constexpr int kUnits = R * 2;  // (4 rows x 8 k) units per tile
  static_assert(kUnits == kProducerThreads, "one unit per producer thread");
  const uint8_t* codes;
  const uint8_t* absmax_q;
  const float* absmax_s2;
  int64_t N, K, k0;
  __device__ __forceinline__ void set_origin(int64_t o) { k0 = o; }
  struct Regs { uint32_t c[4]; uint32_t q8[4]; float s2[4]; };
  __device__ __forceinline__ void load(int step, Regs& r, int t) const {
    const int kc = t % (R / 8), rg = t / (R / 8);
    const int64_t k = k0 + kc * 8;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t n = (int64_t)step * kStep + rg * 4 + e;
      if (n < N && k < K) {
        const int64_t el = n * K + k;
        r.c[e] = *reinterpret_cast<const uint32_t*>(codes + el / 2);
        const int64_t b = el / kBlock;
        r.q8[e] = absmax_q[b];
        r.s2[e] = absmax_s2[b / kGroup];
      } else {
        r.c[e] = 0x77777777u;
        r.q8[e] = 0;
        r.s2[e] = 0.0f;
      }
    }
  }
  __device__ __forceinline__ void store(const Regs& r, uint16_t* tile, const float* lv, int t) const {
    const int kc = t % (R / 8), rg = t / (R / 8);
    float cs[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) cs[e] = block_scale(r.q8[e], r.s2[e]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = lv[(r.c[e] >> (4 * j)) & 15u] * cs[e];
      st_lds_8(tile + (kc * 8 + j) * kLdsStride + rg * 4,
               u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])});
    }
  }
};

// A segment that is never used.
struct LoadNone {
  struct Regs {};
  __device__ __forceinline__ void set_origin(int64_t) {}
  __device__ __forceinline__ void load(int, Regs&, int) const {}
  __device__ __forceinline__ void store(const Regs&, uint16_t*, const float*, int) const {}
};

// ---------------------------------------------------------------------------
// Epilogues

// bf16 output, row-major [P x Q] with leading dimension ld.
struct EpiBf16 {
  uint16_t* out;
  int64_t ld, P, Q;
  __device__ __forceinline__ void put(int64_t p, int64_t q, float v) const {
    if (p < P && q < Q) out[p * ld + q] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xffffu);
  }
};

// float32 split-K partial: out[split][p][q], dense [P x Q] per split.
struct EpiPartial {
  float* out;
  int64_t P, Q;
  __device__ __forceinline__ void put(int64_t p, int64_t q, float v, int split) const {
    if (p < P && q < Q) out[((int64_t)split * P + p) * Q + q] = v;
  }
};

}  // namespace gemm
}  // namespace qlora

namespace qlora {
namespace gemm {

// Consumer: one 64-wide contraction step on the LDS tiles.
template <int PT, int QT>
struct Consumer {
  static constexpr int WP = PT / 2, WQ = QT / 2;   // wave tile
  static constexpr int BP = WP / 32, BQ = WQ / 32; // 32x32 MFMA blocks per wave
  floatx16 acc[BP][BQ];

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < BP; ++i)
#pragma unroll
      for (int j = 0; j < BQ; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  }

  __device__ __forceinline__ void step(const uint16_t* sA, const uint16_t* sB, int wave, int lane) {
    const int wp = wave >> 1, wq = wave & 1;
    const int r = lane & 31, half = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < kStep / 16; ++kk) {
      const int coff = kk * 16 + half * 8;
      bf16x8 a[BP], b[BQ];
#pragma unroll
      for (int i = 0; i < BP; ++i)
        a[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(sA + (wp * WP + i * 32 + r) * kLdsStride + coff));
#pragma unroll
      for (int j = 0; j < BQ; ++j)
        b[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(sB + (wq * WQ + j * 32 + r) * kLdsStride + coff));
#pragma unroll
      for (int i = 0; i < BP; ++i)
#pragma unroll
        for (int j = 0; j < BQ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }

  // Visit every accumulator element with its (p, q) tile coordinates.
  template <class F>
  __device__ __forceinline__ void for_each(int wave, int lane, F&& f) const {
    const int wp = wave >> 1, wq = wave & 1;
#pragma unroll
    for (int i = 0; i < BP; ++i)
#pragma unroll
      for (int j = 0; j < BQ; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int p = wp * WP + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
          const int q = wq * WQ + j * 32 + (lane & 31);
          f(p, q, acc[i][j][v]);
        }
  }
};

// The kernel body shared by every contraction.
//   grid.x = nP * nQ * splits, tile order: p fastest, then q, then split.
//   Steps of the first segment: [0, S1); second segment: [S1, S1 + S2).
//   A split covers a contiguous range of the combined steps.
template <int PT, int QT, class LA1, class LB1, class LA2, class LB2, class Epi>
struct Contraction {
  LA1 a1; LB1 b1; LA2 a2; LB2 b2; Epi epi;
  int nP, nQ, splits, S1, S2, steps_per_split;
};

// Producer side of one segment: steps [lo, hi) of the segment's own
// numbering (local step = global step - seg0), with global iteration index
// it0 for the first of them. Step `it` is stored into stage it&1 and is
// followed by exactly one barrier. Loads run two steps ahead in two register
// slots that are only named by compile-time constants.
template <class LA, class LB>
__device__ __forceinline__ void produce_segment(const LA& la, const LB& lb, int lo, int hi,
                                                int it0, uint16_t* smem, int stage_elems,
                                                int a_rows, const float* lv, int t) {
  const int L = hi - lo;
  if (L <= 0) return;
  typename LA::Regs ra0, ra1;
  typename LB::Regs rb0, rb1;
  la.load(lo, ra0, t); lb.load(lo, rb0, t);
  if (L > 1) { la.load(lo + 1, ra1, t); lb.load(lo + 1, rb1, t); }
  for (int i = 0; i < L; i += 2) {
    {
      uint16_t* sA = smem + ((it0 + i) & 1) * stage_elems;
      la.store(ra0, sA, lv, t);
      lb.store(rb0, sA + a_rows * kLdsStride, lv, t);
      if (i + 2 < L) { la.load(lo + i + 2, ra0, t); lb.load(lo + i + 2, rb0, t); }
    }
    __syncthreads();
    if (i + 1 >= L) break;
    {
      uint16_t* sA = smem + ((it0 + i + 1) & 1) * stage_elems;
      la.store(ra1, sA, lv, t);
      lb.store(rb1, sA + a_rows * kLdsStride, lv, t);
      if (i + 3 < L) { la.load(lo + i + 3, ra1, t); lb.load(lo + i + 3, rb1, t); }
    }
    __syncthreads();
  }
}

template <int PT, int QT, class LA1, class LB1, class LA2, class LB2, class Epi, bool kPartial>
__global__ void __launch_bounds__(kThreads)
contraction_kernel(Contraction<PT, QT, LA1, LB1, LA2, LB2, Epi> cfg) {
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  __shared__ float s_lv[16];
  constexpr int kStageElems = (PT + QT) * kLdsStride;

  const int tid = threadIdx.x;
  // the role split is per wave: keep it in a scalar register so that each
  // role's barriers are reached only by that role's waves
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  if (tid < 16) s_lv[tid] = kNF4[tid];

  int id = blockIdx.x;
  const int pt = id % cfg.nP; id /= cfg.nP;
  const int qt = id % cfg.nQ; id /= cfg.nQ;
  const int split = id;
  const int total = cfg.S1 + cfg.S2;
  const int s_begin = split * cfg.steps_per_split;
  const int s_end = min(total, s_begin + cfg.steps_per_split);
  const int n = max(0, s_end - s_begin);

  __syncthreads();  // level table visible to every wave

  if (wave < 4) {
    // consumers: n steps, one barrier before each
    Consumer<PT, QT> cons;
    cons.zero();
    for (int it = 0; it < n; ++it) {
      __syncthreads();  // stage it&1 written
      const uint16_t* sA = smem + (it & 1) * kStageElems;
      cons.step(sA, sA + PT * kLdsStride, wave, lane);
    }
    __syncthreads();  // matches the producers' final barrier
    const int64_t p0 = (int64_t)pt * PT, q0 = (int64_t)qt * QT;
    if constexpr (kPartial) {
      cons.for_each(wave, lane, [&](int p, int q, float v) { cfg.epi.put(p0 + p, q0 + q, v, split); });
    } else {
      cons.for_each(wave, lane, [&](int p, int q, float v) { cfg.epi.put(p0 + p, q0 + q, v); });
    }
  } else {
    // producers: store step it, then the barrier the consumers wait on
    const int t = tid - kProducerThreads;
    const int lo1 = s_begin, hi1 = min(s_end, cfg.S1);
    const int lo2 = max(s_begin, cfg.S1), hi2 = s_end;
    {
      LA1 a = cfg.a1; LB1 b = cfg.b1;
      a.set_origin((int64_t)pt * PT); b.set_origin((int64_t)qt * QT);
      produce_segment(a, b, lo1, hi1, 0, smem, kStageElems, PT, s_lv, t);
    }
    {
      LA2 a = cfg.a2; LB2 b = cfg.b2;
      a.set_origin((int64_t)pt * PT); b.set_origin((int64_t)qt * QT);
      produce_segment(a, b, lo2 - cfg.S1, hi2 - cfg.S1, max(0, hi1 - lo1), smem, kStageElems,
                      PT, s_lv, t);
    }
    __syncthreads();  // final
  }
}

}  // namespace gemm
}  // namespace qlora
