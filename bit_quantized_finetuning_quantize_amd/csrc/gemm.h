// Tiled bf16 MFMA contraction with warp-specialized producers.
//
//   C[p][q] = sum_c  Aop[p][c] * Bop[q][c]      (float32 accumulation)
//
// A workgroup owns a PT x QT tile of C and walks the contraction in steps of
// 64. Waves 0-3 are consumers: each holds a (PT/2) x (QT/2) accumulator and
// issues v_mfma_f32_32x32x16_bf16 on operand tiles read from LDS. Waves 4-7
// are producers: they move the operand tiles of the coming steps into a
// three-stage LDS ring, either with direct global->LDS buffer loads (plain
// bf16 rows: no register or VALU cost) or through registers when a tile has
// to be converted (NF4 dequantization, transposition).
//
// LDS tile layout: [rows][64] bf16, 128 bytes per row, the sixteen-byte
// chunk c of row r stored at chunk position c ^ ((r >> 1) & 7). The XOR
// swizzle keeps the 32 rows read by one MFMA fragment load on distinct
// banks, and it is what a direct load produces when lane L of an
// instruction fetches logical chunk (L % 8) ^ swizzle(row).
//
// Producer schedule (first segment): while the consumers work on step it,
// the producers issue the direct loads of step it+2, convert the registers
// of step it+1 into LDS, issue the register loads of step it+3, and wait
// until the direct loads of step it+1 have landed. Every prefetch load is
// issued unconditionally (buffer loads past the end of a tensor return 0
// and their results are never stored), so the vector-memory counter waits
// are exact constants. A second segment (steps S1 .. S1+S2-1, the LoRA
// columns) is produced one step ahead without prefetch.
#pragma once

#include "common.h"

namespace qlora {
namespace gemm {

constexpr int kStep = 64;                 // contraction elements per step
constexpr int kRowBytes = 128;            // one LDS tile row
constexpr int kStages = 3;
constexpr int kProducerThreads = 256;     // 4 producer waves
// Consumer waves per workgroup: 8 (two per SIMD, 64x64 each) for the
// forward's 256-row tiles, whose B loader (Nf4Rows) asks for them: one
// wave's matrix work then covers the other's fragment reads after each
// barrier. 4 (128x64 each) otherwise: the input-gradient kernel measured
// faster with fewer LDS reads, and the low-rank tiles are small.
template <int PT, class LB>
constexpr int cons_waves() { return (PT >= 256 && LB::kWideConsumers) ? 8 : 4; }
template <int PT, class LB>
constexpr int threads_for() { return cons_waves<PT, LB>() * 64 + kProducerThreads; }

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }
// byte offset of logical 16-byte chunk c of tile row `row`
__device__ __forceinline__ int tile_off(int row, int c) {
  return row * kRowBytes + ((c ^ swz(row)) << 4);
}

// Buffer resource over [base, base + bytes): loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  if (bytes < 0) bytes = 0;
  if (bytes > 0x7ffffff0LL) bytes = 0x7ffffff0LL;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier for the stage ring. Each wave first waits for its own
// LDS stores (lgkmcnt); the direct-load data of a stage is covered by the
// producers' explicit vector-memory waits before this barrier. The asm
// clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Loaders. Interface:
//   kDirect   direct-load instructions per producer wave per step
//   kRegLoads vector-memory register loads per producer thread per step
//   Regs      per-thread registers of one step
//   setup(tile_origin, t)           once per workgroup
//   direct(step, tile, t)           issue direct global->LDS loads
//   load(step, regs, t)             global -> registers
//   store(regs, tile, tables, t)    registers -> LDS
// `step` counts 64-wide contraction steps from the start of the segment;
// `tile` is the LDS byte address of the operand tile of one stage. Loads
// for steps past the end are allowed and harmless.

struct Tables {
  const float* lv;    // 16 levels of the store type (LDS)
  const float* lv16;  // the same levels at a 16-byte stride (LDS)
  const float* l8;    // 256 values of the 8-bit constant code (LDS)
  float klv[16];      // the 16 levels again, wave-uniform (scalar registers)
};

// Rows of a row-major bf16 matrix, contraction contiguous, moved by direct
// loads. Rows at or past `rows` read as zero. The contraction length of the
// segment must be a multiple of 64.
template <int R>
struct DirectRows {
  static constexpr bool kWideConsumers = false;
  static constexpr int kDirect = R / 32;  // 1 KiB (8 rows) per instruction
  static constexpr int kRegLoads = 0;
  const uint16_t* base;
  int64_t ld;    // elements between rows
  int64_t rows;  // valid rows
  const void* rb; int64_t rn;  // buffer range of this tile (set in setup)
  int voff[kDirect];
  struct Regs {};
  __device__ __forceinline__ void setup(int64_t row0, int t) {
    rb = base + row0 * ld;
    rn = (rows - row0) * ld * 2;
    const int pw = t >> 6, lane = t & 63;
#pragma unroll
    for (int i = 0; i < kDirect; ++i) {
      const int row = (pw * kDirect + i) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ swz(row);
      voff[i] = (int)(row * ld * 2) + c * 16;
    }
  }
  __device__ __forceinline__ void direct(int step, uint32_t tile, int t) const {
    const int pw = t >> 6;
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(rb, rn);
#pragma unroll
    for (int i = 0; i < kDirect; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (lds_void*)(uintptr_t)(tile + (uint32_t)((pw * kDirect + i) * 1024)), 16,
          voff[i], step * (kStep * 2), 0, 0);
  }
  __device__ __forceinline__ void load(int, Regs&, int) const {}
  __device__ __forceinline__ void store(const Regs&, uint32_t, const Tables&, int) const {}
};

// LoRA dropout keep bits (row-major [rows][ld] words, bit j of word w is
// column 32 w + j) as AND masks over eight bf16 values: bit i of `bits`
// keeps element i, i.e. half (i & 1) of word i / 2.
__device__ __forceinline__ u32x4 keep_mask8(uint32_t bits) {
  u32x4 m;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t lo = 0u - ((bits >> (2 * w)) & 1u);
    const uint32_t hi = 0u - ((bits >> (2 * w + 1)) & 1u);
    m[w] = (lo & 0xffffu) | (hi & 0xffff0000u);
  }
  return m;
}

// Rows of a row-major bf16 matrix with a dropout keep mask applied on the
// way into LDS (dropped elements become +0): through registers, one unit is
// 16 contraction elements of one row. Rows at or past `rows` read as zero.
template <int R>
struct MaskedRows {
  static constexpr bool kWideConsumers = false;
  static constexpr int kUnits = R * 4;
  static constexpr int kPer = (kUnits + kProducerThreads - 1) / kProducerThreads;
  static constexpr int kDirect = 0;
  static constexpr int kRegLoads = 3 * kPer;
  const uint16_t* base;
  int64_t ld;    // elements between rows
  int64_t rows;  // valid rows
  const uint32_t* mask;  // keep bits, [rows][mld] words
  int64_t mld;
  const void* rb; int64_t rn; const void* mb; int64_t mn;
  int voff[kPer], moff[kPer];
  struct Regs { u32x4 x[kPer][2]; uint32_t m[kPer]; };
  __device__ __forceinline__ void setup(int64_t row0, int t) {
    rb = base + row0 * ld;
    rn = (rows - row0) * ld * 2;
    mb = mask + row0 * mld;
    mn = (rows - row0) * mld * 4;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int id = t + u * kProducerThreads;
      const int row = id >> 2, q = id & 3;
      const bool ok = id < kUnits;
      voff[u] = ok ? (int)(row * ld * 2) + q * 32 : 0x7ffffff0;
      moff[u] = ok ? (int)(row * mld * 4) + (q >> 1) * 4 : 0x7ffffff0;
    }
  }
  __device__ __forceinline__ void direct(int, uint32_t, int) const {}
  __device__ __forceinline__ void load(int step, Regs& r, int) const {
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(rb, rn);
    const __amdgpu_buffer_rsrc_t msrc = make_rsrc(mb, mn);
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
#pragma unroll
      for (int c = 0; c < 2; ++c)
        r.x[u][c] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff[u] + c * 16, step * (kStep * 2), 0));
      r.m[u] = __builtin_amdgcn_raw_buffer_load_b32(msrc, moff[u], step * (kStep / 8), 0);
    }
  }
  __device__ __forceinline__ void store(const Regs& r, uint32_t tile, const Tables&, int t) const {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int id = t + u * kProducerThreads;
      if (id >= kUnits) continue;
      const int row = id >> 2, q = id & 3;
      const uint32_t bits = r.m[u] >> ((q & 1) * 16);
#pragma unroll
      for (int c = 0; c < 2; ++c)
        *(lds_u32x4*)(uintptr_t)(tile + (uint32_t)tile_off(row, 2 * q + c)) =
            r.x[u][c] & keep_mask8(bits >> (8 * c));
    }
  }
};

// Transposed bf16 source through registers: tile row i = source column
// col0 + i, contraction = source row. Each unit is 4 source rows x 8 source
// columns. Source rows at or past `rows` read as zero. With kMask, a
// dropout keep mask over the source ([rows][mld] words) zeroes the dropped
// elements; a null mask keeps everything.
template <int R, bool kMask = false>
struct ColsBf16 {
  static constexpr bool kWideConsumers = false;
  static constexpr int kUnits = R * 2;
  static constexpr int kPer = (kUnits + kProducerThreads - 1) / kProducerThreads;
  static constexpr int kDirect = 0;
  static constexpr int kRegLoads = (kMask ? 8 : 4) * kPer;
  const uint16_t* base;
  int64_t ld;    // elements between source rows
  int64_t rows;  // valid source rows (contraction length)
  int64_t cols;  // valid source columns
  const uint32_t* mask;  // kMask only: keep bits of the source, or null
  int64_t mld;
  const void* rb; int64_t rn; const void* mb; int64_t mn;
  uint32_t mor;  // all ones when there is no mask
  int voff[kPer], moff[kPer];
  struct Regs { u32x4 v[kPer][4]; uint32_t m[kMask ? kPer : 1][4]; };
  __device__ __forceinline__ void setup(int64_t col0, int t) {
    rb = base + col0;
    rn = rows * ld * 2 - col0 * 2;
    if constexpr (kMask) {
      mb = mask ? mask + (col0 >> 5) : nullptr;
      mn = mask ? rows * mld * 4 - (col0 >> 5) * 4 : 0;
      mor = mask ? 0u : 0xffffffffu;
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int id = t + u * kProducerThreads;
      const int rg = id % (R / 8), cg = id / (R / 8);
      const bool ok = id < kUnits && col0 + rg * 8 < cols;
      voff[u] = ok ? (int)((cg * 4) * ld * 2 + rg * 16) : 0x7ffffff0;
      if constexpr (kMask) moff[u] = ok ? (int)((cg * 4) * mld * 4 + (rg >> 2) * 4) : 0x7ffffff0;
    }
  }
  __device__ __forceinline__ void direct(int, uint32_t, int) const {}
  __device__ __forceinline__ void load(int step, Regs& r, int) const {
    const int soff = (int)((int64_t)step * kStep * ld * 2);
    const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(rb, rn);
#pragma unroll
    for (int u = 0; u < kPer; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        r.v[u][e] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff[u] + (int)(e * ld * 2), soff, 0));
    if constexpr (kMask) {
      const int msoff = (int)((int64_t)step * kStep * mld * 4);
      const __amdgpu_buffer_rsrc_t msrc = make_rsrc(mb, mn);
#pragma unroll
      for (int u = 0; u < kPer; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          r.m[u][e] = __builtin_amdgcn_raw_buffer_load_b32(msrc, moff[u] + (int)(e * mld * 4), msoff, 0);
    }
  }
  __device__ __forceinline__ void store(const Regs& r_in, uint32_t tile, const Tables&, int t) const {
    Regs r = r_in;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int id = t + u * kProducerThreads;
      if (id >= kUnits) continue;
      const int rg = id % (R / 8), cg = id / (R / 8);
      if constexpr (kMask) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          r.v[u][e] &= keep_mask8(((r.m[u][e] | mor) >> ((rg & 3) * 8)) & 0xffu);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1, sh = (e & 1) * 16;
        const uint32_t a0 = (r.v[u][0][w] >> sh) & 0xffffu;
        const uint32_t a1 = (r.v[u][1][w] >> sh) & 0xffffu;
        const uint32_t a2 = (r.v[u][2][w] >> sh) & 0xffffu;
        const uint32_t a3 = (r.v[u][3][w] >> sh) & 0xffffu;
        const uint32_t a = tile + (uint32_t)(tile_off(rg * 8 + e, cg >> 1) + (cg & 1) * 8);
        *(lds_u32x2*)(uintptr_t)a = u32x2{a0 | (a1 << 16), a2 | (a3 << 16)};
      }
    }
  }
};

// Where the two NF4 loaders find a block's constant. With double
// quantization: 8-bit code absmax_q[b] and second-level constant
// absmax_s2[b >> 8]. Without it (absmax_q null): absmax_s2[b] is the float32
// constant itself, read through the same path with the group shift 0 and the
// 8-bit code forced to 255, since fl(fl(255/255) c) = fl(1 c) = c exactly.
struct Nf4Consts {
  int gshift = 8;      // log2 of the blocks per second-level constant
  uint32_t q8or = 0u;  // 255 without double quantization
  __device__ __forceinline__ int64_t s2_bytes(int64_t nblocks) const {
    return ((nblocks + (1ll << gshift) - 1) >> gshift) * 4;
  }
};

// NF4 weight rows (forward): tile row i = weight row n0 + i (output
// feature), contraction = input feature k; a step is one 64-block of each
// row. Two producer threads per row, 32 codes each.
template <int R>
struct Nf4Rows {
  static constexpr bool kWideConsumers = true;
  static_assert(R * 2 == kProducerThreads, "two producer threads per row");
  static constexpr int kDirect = 0;
  static constexpr int kRegLoads = 3;
  const uint8_t* codes;
  const uint8_t* absmax_q;
  const float* absmax_s2;
  int64_t N, K;
  Nf4Consts cst;
  int64_t n0_;
  int vcode, vq;
  int blk0;  // block index of this thread's row at step 0 (< 2^31 by API limits)
  struct Regs { u32x4 c; uint32_t q8; float s2; };
  __device__ __forceinline__ void setup(int64_t n0, int t) {
    const int row = t >> 1, half = t & 1;
    n0_ = n0;
    vcode = (int)(row * (K / 2)) + half * 16;
    vq = (int)(row * (K / kBlock));
    blk0 = (int)((n0 + row) * (K / kBlock));
  }
  __device__ __forceinline__ void direct(int, uint32_t, int) const {}
  __device__ __forceinline__ void load(int step, Regs& r, int) const {
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(codes + n0_ * (K / 2), (N - n0_) * (K / 2));
    const __amdgpu_buffer_rsrc_t rq =
        absmax_q ? make_rsrc(absmax_q + n0_ * (K / kBlock), (N - n0_) * (K / kBlock))
                 : make_rsrc(nullptr, 0);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(absmax_s2, cst.s2_bytes(N * K / kBlock));
    r.c = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, vcode, step * 32, 0));
    r.q8 = __builtin_amdgcn_raw_buffer_load_b8(rq, vq, step, 0) | cst.q8or;
    const int g = (blk0 + step) >> cst.gshift;
    r.s2 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, g * 4, 0, 0));
  }
  __device__ __forceinline__ void store(const Regs& r, uint32_t tile, const Tables& tb, int t) const {
#pragma clang fp contract(off)
    // lookups by v_perm: the forward's consumers are bound by LDS
    // bandwidth, so the producers keep their level lookups out of it
    const int row = t >> 1, half = t & 1;
    const PermTable pt = perm_table(tb.l8[r.q8] * r.s2, tb.klv);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t a = tile + (uint32_t)tile_off(row, half * 4 + w);
      *(lds_u32x4*)(uintptr_t)a = dequant_word_perm(r.c[w], pt);
    }
  }
};

// NF4 weight, transposed (input gradient): tile row i = input feature
// k0 + i, contraction = output feature n. Producer lane t owns the weight
// rows n = 64 step + 2 (t % 32) and the next one, and input features
// k0 + 16 (t / 32) .. + 15 (one 8-byte code load per row, inside one
// 64-block, with the row's 8-bit and second-level constants). For each k
// the lane writes the two rows' values as one 4-byte store, and the 32 lanes
// of a half-wave fill one whole 128-byte LDS row: 16 stores per lane and
// step, each without bank conflicts inside a half-wave.
template <int R>
struct Nf4Cols {
  static constexpr bool kWideConsumers = false;
  static_assert(R == 128, "eight groups of 16 tile rows");
  static constexpr int kDirect = 0;
  static constexpr int kRegLoads = 6;
  const uint8_t* codes;
  const uint8_t* absmax_q;
  const float* absmax_s2;
  int64_t N, K;
  Nf4Consts cst;
  int vcode[2], vq[2];
  int blk0[2];  // block index of (row 2 (t % 32) + h, this k range) at step 0
  struct Regs { u32x2 c[2]; uint32_t q8[2]; float s2[2]; };
  __device__ __forceinline__ void setup(int64_t k0, int t) {
    const int np = t & 31, kq = t >> 5;
    const int64_t k = k0 + kq * 16;
    const bool ok = k < K;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t e = (int64_t)(2 * np + h) * K + k;
      vcode[h] = ok ? (int)(e / 2) : 0x7ffffff0;
      vq[h] = ok ? (int)(e / kBlock) : 0x7ffffff0;
      blk0[h] = (int)(e / kBlock);
    }
  }
  __device__ __forceinline__ void direct(int, uint32_t, int) const {}
  __device__ __forceinline__ void load(int step, Regs& r, int) const {
    const __amdgpu_buffer_rsrc_t rc = make_rsrc(codes, (N * K) / 2);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(absmax_q, absmax_q ? (N * K) / kBlock : 0);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(absmax_s2, cst.s2_bytes(N * K / kBlock));
    const int kb = (int)(K / kBlock);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      r.c[h] = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_raw_buffer_load_b64(rc, vcode[h], step * kStep * (int)(K / 2), 0));
      r.q8[h] = __builtin_amdgcn_raw_buffer_load_b8(rq, vq[h], step * kStep * kb, 0) | cst.q8or;
      const int g = (blk0[h] + step * kStep * kb) >> cst.gshift;
      r.s2[h] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, g * 4, 0, 0));
    }
  }
  __device__ __forceinline__ void store(const Regs& r, uint32_t tile, const Tables& tb, int t) const {
#pragma clang fp contract(off)
    // level lookups from LDS: this producer is bound by its transposing
    // stores, and the input-gradient consumers leave LDS bandwidth to spare;
    // all 32 lookups are issued before any use (one LDS round trip)
    const int np = t & 31, kq = t >> 5;
    float lv[2][16];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const CodeOffsets o = code_offsets(r.c[h][w]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          lv[h][8 * w + 2 * j] = level_lo(tb.lv, o, j);
          lv[h][8 * w + 2 * j + 1] = level_hi(tb.lv16, o, j);
        }
      }
    asm volatile("" ::: "memory");
    const float cs0 = tb.l8[r.q8[0]] * r.s2[0];
    const float cs1 = tb.l8[r.q8[1]] * r.s2[1];
    const uint32_t col = (uint32_t)((np & 3) * 4);
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const uint32_t pk = pack_bf16x2(lv[0][kk] * cs0, lv[1][kk] * cs1);
      const uint32_t a = tile + (uint32_t)tile_off(kq * 16 + kk, np >> 2) + col;
      *(__attribute__((address_space(3))) uint32_t*)(uintptr_t)a = pk;
    }
  }
};

// A segment that is never used.
struct LoadNone {
  static constexpr bool kWideConsumers = false;
  static constexpr int kDirect = 0;
  static constexpr int kRegLoads = 0;
  struct Regs {};
  __device__ __forceinline__ void setup(int64_t, int) {}
  __device__ __forceinline__ void direct(int, uint32_t, int) const {}
  __device__ __forceinline__ void load(int, Regs&, int) const {}
  __device__ __forceinline__ void store(const Regs&, uint32_t, const Tables&, int) const {}
};

// ---------------------------------------------------------------------------
// Epilogues

// bf16 output, row-major [P x Q] with leading dimension ld. Written
// through LDS in whole row segments (Consumer::store_bf16_staged).
struct EpiBf16 {
  static constexpr bool kKeepSeg2 = false;
  static constexpr bool kStaged = true;
  uint16_t* out;
  int64_t ld, P, Q;
  __device__ __forceinline__ void put(int64_t p, int64_t q, float v) const {
    if (p < P && q < Q) out[p * ld + q] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xffffu);
  }
};

// bf16 output whose second segment (the LoRA columns) passes through a
// dropout keep mask over the output, [P][mld] words: C = seg1 + keep o seg2.
// The consumers sum the second segment apart from the first and add only
// its kept elements (at most three second-segment steps, one split).
struct EpiBf16Keep {
  static constexpr bool kKeepSeg2 = true;
  static constexpr bool kStaged = false;
  uint16_t* out;
  int64_t ld, P, Q;
  const uint32_t* mask;
  int64_t mld;
  __device__ __forceinline__ void put(int64_t p, int64_t q, float v) const {
    if (p < P && q < Q) out[p * ld + q] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xffffu);
  }
};

// float32 split-K partial: out[split][p][q], dense [P x Q] per split.
struct EpiPartial {
  static constexpr bool kKeepSeg2 = false;
  static constexpr bool kStaged = false;
  float* out;
  int64_t P, Q;
  __device__ __forceinline__ void put(int64_t p, int64_t q, float v, int split) const {
    if (p < P && q < Q) out[((int64_t)split * P + p) * Q + q] = v;
  }
};

// ---------------------------------------------------------------------------
// Consumer: one 64-wide contraction step on the LDS tiles.
template <int PT, int QT, int CW>
struct Consumer {
  static constexpr int WP = PT / (CW / 2), WQ = QT / 2;   // wave tile
  static constexpr int BP = WP / 32, BQ = WQ / 32; // 32x32 MFMA blocks per wave
  floatx16 acc[BP][BQ];
  int a_off[4], b_off[4];  // per-lane LDS byte offsets of sub-step kk, block 0

  __device__ __forceinline__ void init(int wave, int lane) {
    const int wp = wave >> 1, wq = wave & 1;
    const int r = lane & 31, half = lane >> 5;
    // blocks of one wave are 32 rows apart, which leaves the swizzle unchanged
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      a_off[kk] = tile_off(wp * WP + r, 2 * kk + half);
      b_off[kk] = tile_off(wq * WQ + r, 2 * kk + half);
    }
#pragma unroll
    for (int i = 0; i < BP; ++i)
#pragma unroll
      for (int j = 0; j < BQ; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  }

  __device__ __forceinline__ void frags(uint32_t sA, uint32_t sB, int kk, bf16x8 (&a)[BP],
                                        bf16x8 (&b)[BQ]) const {
#pragma unroll
    for (int i = 0; i < BP; ++i)
      a[i] = as_bf16x8(*(const lds_u32x4*)(uintptr_t)(sA + a_off[kk] + i * 32 * kRowBytes));
#pragma unroll
    for (int j = 0; j < BQ; ++j)
      b[j] = as_bf16x8(*(const lds_u32x4*)(uintptr_t)(sB + b_off[kk] + j * 32 * kRowBytes));
  }
  __device__ __forceinline__ void mma(const bf16x8 (&a)[BP], const bf16x8 (&b)[BQ]) {
#pragma unroll
    for (int i = 0; i < BP; ++i)
#pragma unroll
      for (int j = 0; j < BQ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
  // four 16-deep sub-steps; the fragments of sub-step kk+1 are read while
  // the matrix cores work on sub-step kk. One sub-step ahead, not two: right
  // after a stage barrier every consumer wave reads its first fragments at
  // once, and a smaller burst lets the first MFMAs start sooner (same-box
  // A/B: equal or up to 2 % faster, bit-identical).
  __device__ __forceinline__ void step(uint32_t sA, uint32_t sB) {
    bf16x8 a0[BP], b0[BQ], a1[BP], b1[BQ];
    frags(sA, sB, 0, a0, b0);
    mma(a0, b0);
    frags(sA, sB, 1, a1, b1);
    mma(a1, b1);
    frags(sA, sB, 2, a0, b0);
    mma(a0, b0);
    frags(sA, sB, 3, a1, b1);
    mma(a1, b1);
    // the reads of sub-step kk + 1 go out after the first MFMA of kk
    constexpr int kF = BP + BQ, kM = BP * BQ;
    __builtin_amdgcn_sched_group_barrier(0x100, kF, 0);      // LDS reads kk = 0
#pragma unroll
    for (int kk = 0; kk < 3; ++kk) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // first MFMA of kk
      __builtin_amdgcn_sched_group_barrier(0x100, kF, 0);      // LDS reads kk + 1
      __builtin_amdgcn_sched_group_barrier(0x008, kM - 1, 0);  // rest of kk
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kM, 0);      // MFMA kk = 3
  }

  // Keep bits of this lane's accumulator elements under a dropout mask over
  // the output ([rows][mld] words; `mrs` covers the workgroup's rows, `qw`
  // is the word column of the tile's first column): bit v of keep[i][j] is
  // element v of block (i, j). A 64-bit load gives the words of both column
  // blocks of a row. Read before the main loop, whose registers have room
  // for the eight results.
  template <int BPn = BP, int BQn = BQ>
  __device__ __forceinline__ void load_keep(uint32_t (&keep)[BPn][BQn], __amdgpu_buffer_rsrc_t mrs,
                                            int64_t mld, int qw, int wave, int lane) const {
    static_assert(BQn == 2, "two 32-column blocks per wave: one 64-bit word pair per row");
    const int wp = wave >> 1, wq = wave & 1;
    const int wcol = (qw + (wq * WQ) / 32) * 4;
#pragma unroll
    for (int i = 0; i < BPn; ++i) {
      keep[i][0] = 0u;
      keep[i][1] = 0u;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int p = wp * WP + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
        const u32x2 w = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_raw_buffer_load_b64(mrs, (int)(p * mld * 4) + wcol, 0, 0));
        keep[i][0] |= ((w[0] >> (lane & 31)) & 1u) << v;
        keep[i][1] |= ((w[1] >> (lane & 31)) & 1u) << v;
      }
      // packed here, not after the main loop: the loaded words must not
      // stay live across it
      asm volatile("" : "+v"(keep[i][0]), "+v"(keep[i][1]));
    }
  }

  // acc += keep o (sum over the LDS stages `st[0..ns)` of the tile product),
  // one 32-row block at a time: the second segment's sum needs BQ extra
  // accumulators, not BP * BQ.
  __device__ __forceinline__ void add_kept(const uint32_t (&st)[3], int ns,
                                           const uint32_t (&keep)[BP][BQ]) {
#pragma unroll
    for (int i = 0; i < BP; ++i) {
      floatx16 lr[BQ];
#pragma unroll
      for (int j = 0; j < BQ; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) lr[j][v] = 0.0f;
      for (int s = 0; s < ns; ++s) {
        const uint32_t sA = st[s], sB = st[s] + (uint32_t)(PT * kRowBytes);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const bf16x8 a = as_bf16x8(*(const lds_u32x4*)(uintptr_t)(sA + a_off[kk] + i * 32 * kRowBytes));
#pragma unroll
          for (int j = 0; j < BQ; ++j) {
            const bf16x8 b = as_bf16x8(*(const lds_u32x4*)(uintptr_t)(sB + b_off[kk] + j * 32 * kRowBytes));
            lr[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, lr[j], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < BQ; ++j) {
#pragma unroll
        for (int v = 0; v < 16; ++v)
          acc[i][j][v] += ((keep[i][j] >> v) & 1u) ? lr[j][v] : 0.0f;
        // the sum is final here: the adds may not sink into the epilogue,
        // which would keep every block's lr live at once
        asm volatile("" : "+v"(acc[i][j]));
      }
    }
  }

  // bf16 row-major output through a per-wave LDS staging area at `buf`
  // (32 rows at kStagePitch bytes per wave): each 32-row block of the wave's
  // tile is written to LDS as bf16, read back as 16-byte row chunks and
  // stored as whole 128-byte row segments, 8 global stores per block where
  // element stores would take 64. Rows whose stride, alignment or edge does
  // not allow a 16-byte store take 2-byte stores. The values are those of
  // the element-wise epilogue, bit for bit.
  static constexpr int kStagePitch = WQ * 2 + 16;  // 16 bytes of padding per row
  __device__ __forceinline__ void store_bf16_staged(uint16_t* out, int64_t ld, int64_t P,
                                                    int64_t Q, int64_t p0, int64_t q0,
                                                    uint32_t buf, int wave, int lane) const {
    static_assert(WQ == 64, "eight 16-byte chunks per staged row");
    const int wp = wave >> 1, wq = wave & 1;
    const uint32_t wb = buf + (uint32_t)(wave * 32 * kStagePitch);
    const bool vec = (ld & 7) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0;
#pragma unroll
    for (int i = 0; i < BP; ++i) {
      // elements v and v + 1 of a block are rows r and r + 1 of one column
#pragma unroll
      for (int j = 0; j < BQ; ++j)
#pragma unroll
        for (int v = 0; v < 16; v += 2) {
          const uint32_t pk = pack_bf16x2(acc[i][j][v], acc[i][j][v + 1]);
          const int r = (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
          const uint32_t a = wb + (uint32_t)(r * kStagePitch + (j * 32 + (lane & 31)) * 2);
          *(lds_u16*)(uintptr_t)a = (uint16_t)(pk & 0xffffu);
          *(lds_u16*)(uintptr_t)(a + kStagePitch) = (uint16_t)(pk >> 16);
        }
      // the wave's LDS accesses complete in order: these reads see the
      // writes above, and the next block's writes come after them
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int row = k * 8 + (lane >> 3), ch = lane & 7;
        const u32x4 d =
            *(const lds_u32x4*)(uintptr_t)(wb + (uint32_t)(row * kStagePitch + ch * 16));
        const int64_t p = p0 + wp * WP + i * 32 + row;
        const int64_t q = q0 + wq * WQ + ch * 8;
        if (p >= P) continue;
        uint16_t* o = out + p * ld + q;
        if (vec && q + 8 <= Q) {
          *(u32x4*)o = d;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (q + e < Q) o[e] = (uint16_t)(d[e >> 1] >> ((e & 1) * 16));
        }
      }
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

// Launch parameters of one contraction.
//   grid.x = nP * nQ * splits, tile order: p fastest, then q, then split.
//   Steps of the first segment: [0, S1); second segment: [S1, S1 + S2).
//   A split covers a contiguous range of the combined steps.
template <int PT, int QT, class LA1, class LB1, class LA2, class LB2, class Epi>
struct Contraction {
  LA1 a1; LB1 b1; LA2 a2; LB2 b2; Epi epi;
  int nP, nQ, splits, S1, S2, steps_per_split;
  // XCD-aware tile order (0: off): workgroup id runs on XCD id % 8, so
  // workgroups id = x, x + 8, ... take consecutive tiles of an order that
  // walks groups of xgm P-tiles with q outer; each XCD then covers a block
  // of about (nP / (nP / xgm)) P-tiles by a share of the Q-tiles, and both
  // operands are fetched by fewer XCDs. Needs one split, nP*nQ % 8 == 0 and
  // nP % xgm == 0.
  int xgm;
  // levels and 8-bit constant code of a 4-bit weight operand's store type
  Codebook cb = make_codebook(0);
};

template <int PT, int QT>
constexpr size_t lds_bytes() {  // dynamic LDS: the stage ring
  return (size_t)kStages * (PT + QT) * kRowBytes;
}

// One workgroup per compute unit (the LDS ring takes most of the 160 KiB),
// i.e. two or three waves per SIMD: let the register allocator use that.
template <int PT, int QT, class LA1, class LB1, class LA2, class LB2, class Epi, bool kPartial>
__device__ __forceinline__ void contraction_body(const Contraction<PT, QT, LA1, LB1, LA2, LB2, Epi>& cfg,
                                                 int block) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // lookup tables at fixed LDS addresses (the compiler folds them into the
  // instruction offsets); the dynamic LDS holds the stage ring
  __shared__ float s_lv[16];
  __shared__ __attribute__((aligned(16))) float s_lv16[64];
  __shared__ float s_l8[256];
  constexpr int kStageBytes = (PT + QT) * kRowBytes;
  constexpr uint32_t kBOff = PT * kRowBytes;
  const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) uint8_t*)smem);

  const int tid = threadIdx.x;
  // the role split is per wave: keep it in a scalar register so that each
  // role's barriers are reached only by that role's waves
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  if (tid < 256) s_l8[tid] = level8_of(tid, cfg.cb.dq_fp8);
  if (tid < 16) {
    s_lv[tid] = cfg.cb.lv[tid];
    s_lv16[4 * tid] = cfg.cb.lv[tid];
  }

  int id = block;
  int pt, qt, split;
  if (cfg.xgm > 0) {
    const int tiles = cfg.nP * cfg.nQ;
    const int L = (id & 7) * (tiles >> 3) + (id >> 3);
    const int grp = cfg.xgm * cfg.nQ;
    pt = (L / grp) * cfg.xgm + L % cfg.xgm;
    qt = (L % grp) / cfg.xgm;
    split = 0;
  } else {
    pt = id % cfg.nP; id /= cfg.nP;
    qt = id % cfg.nQ; id /= cfg.nQ;
    split = id;
  }
  const int total = cfg.S1 + cfg.S2;
  const int s_begin = split * cfg.steps_per_split;
  const int s_end = min(total, s_begin + cfg.steps_per_split);
  const int n = max(0, s_end - s_begin);

  __syncthreads();  // tables visible to every wave

  auto stage = [&](int it) { return lds0 + (uint32_t)((it % kStages) * kStageBytes); };
  // seg1 steps of this split: local [0, n1); seg2: local [n1, n)
  const int n1 = max(0, min(s_end, cfg.S1) - s_begin);
  const int g0 = s_begin;  // seg1 local step s is global step g0 + s
  // An A operand of seg1 that only takes direct loads is moved by the
  // consumer waves: the loads are vector-memory instructions that issue
  // between their MFMAs, and the producers keep the register path.
  constexpr bool kConsA = LA1::kDirect > 0 && LA1::kRegLoads == 0;

  constexpr int kCW = cons_waves<PT, LB1>();
  if (wave < kCW) {
    // consumers: n steps, one barrier before each. The first four waves
    // (256 threads) also move the A operand of seg1.
    Consumer<PT, QT, kCW> cons;
    cons.init(wave, lane);
    LA1 a1 = cfg.a1;
    const bool mover = wave < 4;
    if constexpr (kConsA) {
      if (mover && n1 > 0) {
        a1.setup((int64_t)pt * PT, tid);
        a1.direct(g0, stage(0), tid);
        if (n1 > 1) a1.direct(g0 + 1, stage(1), tid);
      }
    }
    // with a kept second segment the loop covers the first segment only;
    // the second's stages are summed after the last barrier
    const int nc = Epi::kKeepSeg2 ? n1 : n;
    uint32_t keep[Epi::kKeepSeg2 ? Consumer<PT, QT, kCW>::BP : 1][2];
    if constexpr (Epi::kKeepSeg2) {
      const int64_t kp0 = (int64_t)pt * PT;
      const __amdgpu_buffer_rsrc_t mrs =
          make_rsrc(cfg.epi.mask + kp0 * cfg.epi.mld, (cfg.epi.P - kp0) * cfg.epi.mld * 4);
      cons.load_keep(keep, mrs, cfg.epi.mld, (int)(((int64_t)qt * QT) >> 5), wave, lane);
    }
    for (int it = 0; it < nc; ++it) {
      if constexpr (kConsA) {
        // this wave's A loads of step it have landed (those of it+1 may fly)
        if (mover && it + 1 < n1) wait_vmcnt<LA1::kDirect>();
        else if (mover && it < n1) wait_vmcnt<0>();
      }
      stage_barrier();  // stage it % 3 written
      // stage (it+2) % 3 was last read in step it-1, which every consumer
      // finished before this barrier
      if constexpr (kConsA) {
        if (mover && it + 2 < n1) a1.direct(g0 + it + 2, stage(it + 2), tid);
      }
      const uint32_t sA = stage(it);
      cons.step(sA, sA + kBOff);
    }
    const int64_t p0 = (int64_t)pt * PT, q0 = (int64_t)qt * QT;
    if constexpr (Epi::kKeepSeg2) {
      for (int it = nc; it < n; ++it) stage_barrier();
      // the second segment's stages (at most three) are all still in the
      // ring: nothing is produced after the last barrier
      const uint32_t st[3] = {stage(n1), stage(n1 + 1), stage(n1 + 2)};
      cons.add_kept(st, min(n - n1, 3), keep);
    }
    if constexpr (kPartial) {
      cons.for_each(wave, lane, [&](int p, int q, float v) { cfg.epi.put(p0 + p, q0 + q, v, split); });
    } else if constexpr (Epi::kStaged) {
      // Stage (n+1) % 3 is free once this wave has passed the last barrier
      // (#n-1): every consumer finished reading it (step n-2) before that
      // barrier, and no load writes it afterwards. The only loads that can
      // still be landing are the first segment's past-the-end direct loads,
      // and they fill stage n1 % 3, which is n % 3 without a second segment
      // and is waited for by the producers before it with one. The other
      // consumers may still be reading stage (n-1) % 3.
      static_assert(kCW * 32 * Consumer<PT, QT, kCW>::kStagePitch <= kStageBytes,
                    "staging area inside one stage");
      cons.store_bf16_staged(cfg.epi.out, cfg.epi.ld, cfg.epi.P, cfg.epi.Q, p0, q0, stage(n + 1),
                             wave, lane);
    } else {
      cons.for_each(wave, lane, [&](int p, int q, float v) { cfg.epi.put(p0 + p, q0 + q, v); });
    }
    return;
  }
  if (n == 0) return;

  // ---- producers: exactly n barriers, one after each produced step ----
  const int t = tid - kCW * 64;
  Tables tb{s_lv, s_lv16, s_l8, {}};
#pragma unroll
  for (int i = 0; i < 16; ++i) tb.klv[i] = cfg.cb.lv[i];

  LA2 a2 = cfg.a2; LB2 b2 = cfg.b2;
  auto seg2_step = [&](int s) {  // local step s >= n1, loaded synchronously
    typename LA2::Regs x; typename LB2::Regs y;
    const int gs = s_begin + s - cfg.S1;
    const uint32_t sa = stage(s);
    a2.direct(gs, sa, t); b2.direct(gs, sa + kBOff, t);
    a2.load(gs, x, t); b2.load(gs, y, t);
    wait_vmcnt<0>();
    a2.store(x, sa, tb, t); b2.store(y, sa + kBOff, tb, t);
  };
  if (n1 < n) { a2.setup((int64_t)pt * PT, t); b2.setup((int64_t)qt * QT, t); }

  int it = 0;  // iteration it produces step it+1; step 0 comes from the prologue
  if (n1 > 0) {
    LA1 a1 = cfg.a1; LB1 b1 = cfg.b1;
    if constexpr (!kConsA) a1.setup((int64_t)pt * PT, t);
    b1.setup((int64_t)qt * QT, t);
    constexpr int kReg = LA1::kRegLoads + LB1::kRegLoads;
    constexpr int kDir = (kConsA ? 0 : LA1::kDirect) + LB1::kDirect;
    typename LA1::Regs ra0, ra1;
    typename LB1::Regs rb0, rb1;
    auto a1_direct = [&](int g, uint32_t sa) {
      if constexpr (!kConsA) a1.direct(g, sa, t);
    };

    // prologue: step 0 complete in stage 0; direct loads of step 1; regs 1, 2.
    // Step 1's loads are issued before the wait for step 0, so that the two
    // travel together; loads complete in issue order, so waiting until the
    // newest kDir + kReg are the only ones outstanding covers step 0.
    a1_direct(g0, stage(0)); b1.direct(g0, stage(0) + kBOff, t);
    a1.load(g0, ra0, t); b1.load(g0, rb0, t);
    a1_direct(g0 + 1, stage(1)); b1.direct(g0 + 1, stage(1) + kBOff, t);
    a1.load(g0 + 1, ra1, t); b1.load(g0 + 1, rb1, t);
    wait_vmcnt<kDir + kReg>();
    a1.store(ra0, stage(0), tb, t); b1.store(rb0, stage(0) + kBOff, tb, t);
    a1.load(g0 + 2, ra0, t); b1.load(g0 + 2, rb0, t);
    stage_barrier();  // barrier #0: step 0 ready

    // Iteration i (producing step i+1 < n1) with rA/rB holding step i+1.
    auto iter = [&](int i, typename LA1::Regs& rA, typename LB1::Regs& rB) {
      a1_direct(g0 + i + 2, stage(i + 2)); b1.direct(g0 + i + 2, stage(i + 2) + kBOff, t);
      a1.store(rA, stage(i + 1), tb, t); b1.store(rB, stage(i + 1) + kBOff, tb, t);
      a1.load(g0 + i + 3, rA, t); b1.load(g0 + i + 3, rB, t);
      wait_vmcnt<2 * kReg + kDir>();  // direct loads of step i+1 have landed
    };
    for (; it + 1 < n1 - 1; it += 2) {
      iter(it, ra1, rb1);
      stage_barrier();
      iter(it + 1, ra0, rb0);
      stage_barrier();
    }
    if (it < n1 - 1) {
      iter(it, ra1, rb1);
      stage_barrier();
      ++it;
    }
    // it == n1 - 1 here
  } else {
    seg2_step(0);
    stage_barrier();  // barrier #0
  }
  // tail: seg2 steps it+1 .. n-1, one per iteration
  for (; it < n - 1; ++it) {
    seg2_step(it + 1);
    stage_barrier();
  }
  wait_vmcnt<0>();  // no direct load may outlive the workgroup's LDS
}

template <int PT, int QT, class LA1, class LB1, class LA2, class LB2, class Epi, bool kPartial>
__global__ void __launch_bounds__((threads_for<PT, LB1>()))
    __attribute__((amdgpu_waves_per_eu((threads_for<PT, LB1>() / 256),
                                       (threads_for<PT, LB1>() / 256))))
contraction_kernel(Contraction<PT, QT, LA1, LB1, LA2, LB2, Epi> cfg) {
  contraction_body<PT, QT, LA1, LB1, LA2, LB2, Epi, kPartial>(cfg, blockIdx.x);
}

// Two independent contractions of one shape in one launch: workgroups
// [0, nb0) run c0, the rest run c1.
template <int PT, int QT, class LA1, class LB1, class LA2, class LB2, class Epi, bool kPartial>
__global__ void __launch_bounds__((threads_for<PT, LB1>()))
    __attribute__((amdgpu_waves_per_eu((threads_for<PT, LB1>() / 256),
                                       (threads_for<PT, LB1>() / 256))))
contraction_pair_kernel(Contraction<PT, QT, LA1, LB1, LA2, LB2, Epi> c0,
                        Contraction<PT, QT, LA1, LB1, LA2, LB2, Epi> c1, int nb0) {
  if ((int)blockIdx.x < nb0)
    contraction_body<PT, QT, LA1, LB1, LA2, LB2, Epi, kPartial>(c0, blockIdx.x);
  else
    contraction_body<PT, QT, LA1, LB1, LA2, LB2, Epi, kPartial>(c1, blockIdx.x - nb0);
}

}  // namespace gemm
}  // namespace qlora
