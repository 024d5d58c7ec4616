// Forward (large M) and backward of the NF4 linear layer with a LoRA term.
//
// ozercemkelahmet.com "QLoRA", How it works, Step 5 (dequantize each block
// into the compute type, multiply, add the adapter path) and Step 6
// (gradients reach the adapter through the dequantized product; the frozen
// weight gets none); crackai.dev "QLoRA: Efficient Finetuning of Quantized
// LLMs", Training Flow.
//
// Forward, M > 16:
//   1. T = X A            split-K MFMA contraction -> partials -> reduce,
//                         which also writes bf16(s T) for step 2
//   2. Y = X W'^T + (sT) B   one MFMA contraction over K + r: the frozen
//                         weight is dequantized tile by tile by producer
//                         waves, the adapter columns form a second segment.
// Backward:
//   1. G = dY B^T         split-K contraction -> reduce (fp32 G, bf16 s G,
//                         bf16 (s G)^T)
//   2. bf16 (s T)^T from T (in the same reduce launch), or T recomputed
//      when the caller passes none
//   3. dX = dY W' + (sG) A^T   one contraction over N + r; the weight tile is
//                         dequantized and transposed into LDS
//   4. dA = X^T (sG),  dB = (sT)^T dY   split-M contractions -> reduce
//
// LoRA dropout (ozercemkelahmet.com "QLoRA", the LoraConfig of "A code
// example with common libraries"; "Practical guidance and best practices",
// Adapter settings): the adapter path
// takes D(X) = (X o keep) f, f the inverse keep probability, from a keep
// mask over X. The mask is applied where X enters the T and dA products
// (on the way into LDS) and, for dX, to the LoRA columns' contribution,
// summed apart from the frozen-weight product; f rides on the float32
// reduction of T and G.
#include "common.h"
#include "gemm.h"
#include "kernels.h"

#include <algorithm>
#include <atomic>

namespace qlora {

using namespace gemm;

namespace {

constexpr int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }
constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Number of contraction splits for a split-K launch: at most about one
// workgroup per compute unit (measured faster than two: fewer partials to
// write and sum), at least two steps per split, and among those the count
// whose rounds of 256 workgroups times steps per split is least (ties to
// fewer splits): 118 tiles over 32 steps take 2 splits (236 workgroups, one
// round of 16 steps), not 3 (354 workgroups, two rounds of 11).
int64_t choose_splits(int64_t tiles, int64_t steps) {
  tiles = std::max<int64_t>(tiles, 1);
  const int64_t want = ceil_div(256, tiles);
  const int64_t maxs = std::max<int64_t>(1, steps / 2);
  int64_t best = 1, best_cost = ceil_div(tiles, 256) * steps;
  for (int64_t s = 2; s <= std::min(want, maxs); ++s) {
    const int64_t per = ceil_div(steps, s);
    const int64_t sc = ceil_div(steps, per);  // splits actually formed
    const int64_t cost = ceil_div(tiles * sc, 256) * per;
    if (cost < best_cost) {
      best = sc;
      best_cost = cost;
    }
  }
  return best;
}

// Split count shared by the dA and dB^T contractions of one launch.
int64_t grad_splits(int64_t M, int64_t N, int64_t K, int64_t r64) {
  return choose_splits((ceil_div(K, 128) + ceil_div(N, 128)) * (r64 / 64), ceil_div(M, 64));
}

// ---------------------------------------------------------------------------
// workspace carve-up (byte offsets, 256-aligned)
struct WsLayout {
  int64_t r64, Mp;
  size_t apad, at, t32, st, stt, sg, sgt, part, total;
};

WsLayout ws_layout(int64_t M, int64_t N, int64_t K, int r) {
  WsLayout w{};
  w.r64 = round_up(r, 64);
  w.Mp = round_up(M, 64);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += (bytes + 255) / 256 * 256; return o; };
  w.apad = take((size_t)K * w.r64 * 2);
  w.at = take((size_t)w.r64 * K * 2);
  w.t32 = take((size_t)M * r * 4);
  w.st = take((size_t)w.Mp * w.r64 * 2);
  w.stt = take((size_t)w.r64 * w.Mp * 2);
  w.sg = take((size_t)w.Mp * w.r64 * 2);
  w.sgt = take((size_t)w.r64 * w.Mp * 2);
  // split-K partials: the largest of the four low-rank contractions
  size_t pe = 0;
  auto consider = [&](int64_t P, int64_t Q, int64_t splits) {
    pe = std::max(pe, (size_t)(P * Q * splits));
  };
  consider(M, w.r64, choose_splits(ceil_div(M, 64) * (w.r64 / 64), ceil_div(K, 64)));
  consider(M, w.r64, choose_splits(ceil_div(M, 64) * (w.r64 / 64), ceil_div(N, 64)));
  {  // dA and dB^T partials side by side (one launch, common split count s).
     // With t tiles, s <= 256 / t + 1 and t >= (K + N) r64 / (128 * 64), so
     // the bound below holds for every s and grows with K and N: a workspace
     // sized for the largest shape serves the smaller ones.
    const int64_t sp = grad_splits(M, N, K, w.r64);
    const int64_t bound = 256 * 128 * 64 + (K + N) * w.r64;
    pe = std::max(pe, (size_t)std::max((K + N) * w.r64 * sp, bound));
  }
  // the small-M forward path keeps its own partials here too
  pe = std::max(pe, (size_t)gemv_partial_elems(M, N, K, r));
  w.part = take(pe * 4);
  w.total = off;
  return w;
}

}  // namespace

// Every contraction used below, instantiated explicitly so that the host
// side always emits its launch stub.
namespace gemm {
template __global__ void contraction_kernel<256, 128, DirectRows<256>, Nf4Rows<128>,
    DirectRows<256>, ColsBf16<128>, EpiBf16, false>(
    Contraction<256, 128, DirectRows<256>, Nf4Rows<128>, DirectRows<256>, ColsBf16<128>, EpiBf16>);
template __global__ void contraction_kernel<256, 128, DirectRows<256>, Nf4Cols<128>,
    DirectRows<256>, DirectRows<128>, EpiBf16, false>(
    Contraction<256, 128, DirectRows<256>, Nf4Cols<128>, DirectRows<256>, DirectRows<128>, EpiBf16>);
template __global__ void contraction_kernel<64, 64, DirectRows<64>, DirectRows<64>, LoadNone,
    LoadNone, EpiPartial, true>(
    Contraction<64, 64, DirectRows<64>, DirectRows<64>, LoadNone, LoadNone, EpiPartial>);
template __global__ void contraction_kernel<64, 64, DirectRows<64>, ColsBf16<64>, LoadNone,
    LoadNone, EpiPartial, true>(
    Contraction<64, 64, DirectRows<64>, ColsBf16<64>, LoadNone, LoadNone, EpiPartial>);
template __global__ void contraction_pair_kernel<128, 64, ColsBf16<128>, DirectRows<64>, LoadNone,
    LoadNone, EpiPartial, true>(
    Contraction<128, 64, ColsBf16<128>, DirectRows<64>, LoadNone, LoadNone, EpiPartial>,
    Contraction<128, 64, ColsBf16<128>, DirectRows<64>, LoadNone, LoadNone, EpiPartial>, int);
// with LoRA dropout
template __global__ void contraction_kernel<256, 128, DirectRows<256>, Nf4Cols<128>,
    DirectRows<256>, DirectRows<128>, EpiBf16Keep, false>(
    Contraction<256, 128, DirectRows<256>, Nf4Cols<128>, DirectRows<256>, DirectRows<128>, EpiBf16Keep>);
template __global__ void contraction_kernel<64, 64, MaskedRows<64>, DirectRows<64>, LoadNone,
    LoadNone, EpiPartial, true>(
    Contraction<64, 64, MaskedRows<64>, DirectRows<64>, LoadNone, LoadNone, EpiPartial>);
template __global__ void contraction_kernel<64, 64, MaskedRows<64>, ColsBf16<64>, LoadNone,
    LoadNone, EpiPartial, true>(
    Contraction<64, 64, MaskedRows<64>, ColsBf16<64>, LoadNone, LoadNone, EpiPartial>);
template __global__ void contraction_pair_kernel<128, 64, ColsBf16<128, true>, DirectRows<64>,
    LoadNone, LoadNone, EpiPartial, true>(
    Contraction<128, 64, ColsBf16<128, true>, DirectRows<64>, LoadNone, LoadNone, EpiPartial>,
    Contraction<128, 64, ColsBf16<128, true>, DirectRows<64>, LoadNone, LoadNone, EpiPartial>, int);
}  // namespace gemm

size_t linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int r) {
  return ws_layout(M, N, K, r).total;
}

namespace {

// ---------------------------------------------------------------------------
// small kernels

// Apad[k][j] = A[k][j] for j < r, 0 for r <= j < r64; At = Apad^T [r64 x K].
__global__ void adapter_prep_kernel(const uint16_t* __restrict__ A, int64_t K, int r,
                                    int64_t r64, uint16_t* __restrict__ apad,
                                    uint16_t* __restrict__ at) {
  const int64_t total = K * r64;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t k = i / r64, j = i % r64;
    const uint16_t v = (j < r) ? A[k * r + j] : (uint16_t)0;
    apad[i] = v;
    at[j * K + k] = v;
  }
}

hipError_t prep_adapter(const uint16_t* A, int64_t K, int r, const WsLayout& w, char* ws,
                        hipStream_t stream);

// Reduce split-K partials of an [M x r] low-rank product (partial layout
// [split][M][ld]) and emit, with V = f * (sum of the partials): float32 V
// (optional), bf16(s V) padded [Mp x r64] (optional) and its transpose
// [r64 x Mp] (optional). f is the dropout keep scale (exactly 1 without
// dropout, which leaves the sum unchanged).
struct LowrankJob {
  const float* part;
  int splits;
  int64_t ld;
  float* out32;
  uint16_t* sv;
  uint16_t* svt;
  float f = 1.0f;
};

// One or two jobs of the same shape in one launch (the second one when
// jobs[1].part is set): elements [0, Mp r64) are job 0's, the rest job 1's.
__global__ void reduce_lowrank_kernel(LowrankJob j0, LowrankJob j1, int64_t M, int r,
                                      int64_t r64, int64_t Mp, float s) {
  const int64_t per = Mp * r64;
  const int64_t total = j1.part ? 2 * per : per;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const bool second = i >= per;
    const LowrankJob& jb = second ? j1 : j0;
    const int64_t e = second ? i - per : i;
    const int64_t m = e / r64, j = e % r64;
    float v = 0.0f;
    if (m < M && j < r) {
      for (int sp = 0; sp < jb.splits; ++sp) v += jb.part[((int64_t)sp * M + m) * jb.ld + j];
      v *= jb.f;
      if (jb.out32) jb.out32[m * r + j] = v;
    }
    const uint16_t b = (uint16_t)(pack_bf16x2(s * v, 0.0f) & 0xffffu);
    if (jb.sv) jb.sv[e] = b;
    if (jb.svt) jb.svt[j * Mp + m] = b;
  }
}

// Adapter gradients from their split partials, summed in split order:
//   dA[k][j] = sum_s pa[s][k][j]        (pa dense [splits][K][r64])
//   dB[j][n] = sum_s pb[s][n][j]        (pb dense [splits][N][r64], dB^T)
// One thread per four columns of a partial row (k, then n): consecutive
// threads read consecutive 16-byte pieces of a row.
__global__ void reduce_grads_kernel(const float* __restrict__ pa, const float* __restrict__ pb,
                                    int splits, int64_t K, int64_t N, int r, int64_t r64,
                                    float* __restrict__ dA, float* __restrict__ dB) {
  const int64_t per_row = r64 / 4;
  const int64_t total = (K + N) * per_row;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / per_row;
    const int j0 = (int)(i % per_row) * 4;
    if (j0 >= r) continue;
    const bool is_a = row < K;
    const int64_t p = is_a ? row : row - K;
    const int64_t P = is_a ? K : N;
    const float* part = is_a ? pa : pb;
    floatx4 v = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int sp = 0; sp < splits; ++sp) {
      const floatx4 u = *reinterpret_cast<const floatx4*>(part + ((int64_t)sp * P + p) * r64 + j0);
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] += u[c];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (j0 + c < r) {
        if (is_a) dA[p * r + j0 + c] = v[c];
        else dB[(int64_t)(j0 + c) * N + p] = v[c];
      }
    }
  }
}

unsigned grid_for(int64_t total, int threads = 256) {
  int64_t b = ceil_div(total, threads);
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(b, 8192));
}

// ---------------------------------------------------------------------------
// launching a contraction

// Dynamic LDS above the default limit: raised once per device and kernel
// (the flag is per kernel instantiation), not on every launch.
template <class Kern>
hipError_t raise_lds_limit(Kern kern, size_t lds) {
  static std::atomic<uint64_t> raised{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (raised.load(std::memory_order_acquire) & bit) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e == hipSuccess) raised.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

template <int PT, int QT, class LA1, class LB1, class LA2, class LB2, class Epi, bool kPartial>
hipError_t run(Contraction<PT, QT, LA1, LB1, LA2, LB2, Epi> cfg, hipStream_t stream) {
  auto kern = contraction_kernel<PT, QT, LA1, LB1, LA2, LB2, Epi, kPartial>;
  const size_t lds = lds_bytes<PT, QT>();
  hipError_t e = raise_lds_limit(kern, lds);
  if (e != hipSuccess) return e;
  const int64_t blocks = (int64_t)cfg.nP * cfg.nQ * cfg.splits;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(threads_for<PT, LB1>()), lds, stream, cfg);
  return hipGetLastError();
}

template <int PT, int QT, class LA1, class LB1, class LA2, class LB2, class Epi, bool kPartial>
hipError_t run_pair(Contraction<PT, QT, LA1, LB1, LA2, LB2, Epi> c0,
                    Contraction<PT, QT, LA1, LB1, LA2, LB2, Epi> c1, hipStream_t stream) {
  auto kern = contraction_pair_kernel<PT, QT, LA1, LB1, LA2, LB2, Epi, kPartial>;
  const size_t lds = lds_bytes<PT, QT>();
  hipError_t e = raise_lds_limit(kern, lds);
  if (e != hipSuccess) return e;
  const int64_t nb0 = (int64_t)c0.nP * c0.nQ * c0.splits;
  const int64_t nb1 = (int64_t)c1.nP * c1.nQ * c1.splits;
  hipLaunchKernelGGL(kern, dim3((unsigned)(nb0 + nb1)), dim3(threads_for<PT, LB1>()), lds, stream,
                     c0, c1, (int)nb0);
  return hipGetLastError();
}

// XCD-aware tile order for a one-split launch, when the tile count divides
// among the 8 XCDs: groups of 2 P-tiles, so that the 32 tiles an XCD runs at
// once are 2 P-tiles by 16 Q-tiles. Over a tile's walk along the
// contraction its row operand (256 rows of bf16) is about 7.8 times the
// bytes of its 4-bit weight tile (128 rows), and a round fetches p row
// tiles and 32 / p weight tiles: fewest bytes near p = sqrt(32 / 7.8) = 2
// (measured on the prefill projections: 21 % fewer bytes fetched by the
// forward and 19 % by dX than with groups of half the P-tiles, same time).
template <class C>
void set_xcd_order(C& cfg) {
  cfg.xgm = 0;
  if (cfg.splits == 1 && ((int64_t)cfg.nP * cfg.nQ) % 8 == 0 && cfg.nP % 2 == 0)
    cfg.xgm = 2;
}

template <class C>
void set_steps(C& cfg, int64_t S1, int64_t S2, int64_t tiles) {
  cfg.S1 = (int)S1;
  cfg.S2 = (int)S2;
  const int64_t total = S1 + S2;
  const int64_t splits = choose_splits(tiles, total);
  cfg.steps_per_split = (int)ceil_div(total, splits);
  cfg.splits = (int)ceil_div(total, cfg.steps_per_split);
}

// Low-rank product V[M x r] = Aop[M x C] * Bop[r x C]^T with split-K partials.
// Aop rows come from a bf16 row-major source (DirectRows, or MaskedRows
// under dropout), contraction length C.
template <class LA, class LB>
hipError_t lowrank_partials(LA la, int64_t M, int64_t C, LB lb, int64_t r64, float* part,
                            int* splits_out, hipStream_t stream) {
  Contraction<64, 64, LA, LB, LoadNone, LoadNone, EpiPartial> cfg{};
  cfg.a1 = la;
  cfg.b1 = lb;
  cfg.nP = (int)ceil_div(M, 64);
  cfg.nQ = (int)(r64 / 64);
  set_steps(cfg, ceil_div(C, 64), 0, (int64_t)cfg.nP * cfg.nQ);
  cfg.epi = EpiPartial{part, M, r64};
  *splits_out = cfg.splits;
  return run<64, 64, LA, LB, LoadNone, LoadNone, EpiPartial, true>(cfg, stream);
}

// The loaders' constant mode: double-quantized, or one float32 constant
// per block when the store has no 8-bit codes.
Nf4Consts nf4_consts(const Nf4Weight& W) {
  Nf4Consts c;
  if (!W.absmax_q) {
    c.gshift = 0;
    c.q8or = 255u;
  }
  return c;
}

#define QLORA_TRY(x)                       \
  do {                                     \
    hipError_t e_ = (x);                   \
    if (e_ != hipSuccess) return e_;       \
  } while (0)

// The adapter can be read in place when its rows are whole 64-column tiles
// and 16-byte aligned: no padded copy, no transposed copy.
bool adapter_in_place(const uint16_t* A, int r) {
  return r % 64 == 0 && (reinterpret_cast<uintptr_t>(A) & 15) == 0;
}

hipError_t prep_adapter(const uint16_t* A, int64_t K, int r, const WsLayout& w, char* ws,
                        hipStream_t stream) {
  if (adapter_in_place(A, r)) return hipSuccess;
  hipLaunchKernelGGL(adapter_prep_kernel, dim3(grid_for(K * w.r64)), dim3(256), 0, stream, A, K,
                     r, w.r64, reinterpret_cast<uint16_t*>(ws + w.apad),
                     reinterpret_cast<uint16_t*>(ws + w.at));
  return hipGetLastError();
}

template <class LA>
hipError_t T_partials(LA la, const uint16_t* A, int64_t M, int64_t K, int r, const WsLayout& w,
                      char* ws, float* part, int* splits, hipStream_t stream) {
  if (adapter_in_place(A, r)) {
    // Bop[j][k] = A[k][j]: columns of the adapter, transposed on the way in
    ColsBf16<64> lb{A, (int64_t)r, K, (int64_t)r};
    return lowrank_partials(la, M, K, lb, w.r64, part, splits, stream);
  }
  // Bop[j][k] = A^T[j][k]: rows of the transposed, padded adapter copy
  DirectRows<64> lb{reinterpret_cast<const uint16_t*>(ws + w.at), K, w.r64};
  return lowrank_partials(la, M, K, lb, w.r64, part, splits, stream);
}

// T = D(X) A -> out32 (optional), bf16(s T) [Mp x r64], bf16(s T)^T
// (optional); D(X) = X without dropout (dr.mask null).
hipError_t compute_T(const uint16_t* X, const uint16_t* A, int64_t M, int64_t K, int r,
                     const WsLayout& w, char* ws, float s, float* out32, bool transposed,
                     const Dropout& dr, hipStream_t stream) {
  float* part = reinterpret_cast<float*>(ws + w.part);
  int splits = 0;
  if (dr.mask)
    QLORA_TRY(T_partials(MaskedRows<64>{X, K, M, dr.mask, K / 32}, A, M, K, r, w, ws, part,
                         &splits, stream));
  else
    QLORA_TRY(T_partials(DirectRows<64>{X, K, M}, A, M, K, r, w, ws, part, &splits, stream));
  LowrankJob jt{part, splits, w.r64, out32, reinterpret_cast<uint16_t*>(ws + w.st),
                transposed ? reinterpret_cast<uint16_t*>(ws + w.stt) : nullptr};
  if (dr.mask) jt.f = dr.keep_scale;
  hipLaunchKernelGGL(reduce_lowrank_kernel, dim3(grid_for(w.Mp * w.r64)), dim3(256), 0, stream,
                     jt, LowrankJob{}, M, r, w.r64, w.Mp, s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_gemm(const uint16_t* X, Nf4Weight W, const uint16_t* A,
                           const uint16_t* B, int64_t M, int64_t N, int64_t K, int r,
                           float scale, uint16_t* Y, float* T_out, void* ws_,
                           hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1, Dropout dr) {
  char* ws = reinterpret_cast<char*>(ws_);
  const WsLayout w = ws_layout(M, N, K, r);
  QLORA_TRY(prep_adapter(A, K, r, w, ws, stream));
  float* t32 = T_out ? T_out : reinterpret_cast<float*>(ws + w.t32);
  QLORA_TRY(compute_T(X, A, M, K, r, w, ws, scale, t32, false, dr, stream));

  using LA1 = DirectRows<256>;
  using LB1 = Nf4Rows<128>;
  using LA2 = DirectRows<256>;
  using LB2 = ColsBf16<128>;
  Contraction<256, 128, LA1, LB1, LA2, LB2, EpiBf16> cfg{};
  cfg.a1 = LA1{X, K, M};
  cfg.b1 = LB1{W.codes, W.absmax_q, W.absmax_s2, N, K, nf4_consts(W)};
  cfg.a2 = LA2{reinterpret_cast<const uint16_t*>(ws + w.st), w.r64, M};
  cfg.b2 = LB2{B, N, (int64_t)r, N};  // Bop[n][j] = B[j][n]
  cfg.nP = (int)ceil_div(M, 256);
  cfg.nQ = (int)ceil_div(N, 128);
  cfg.S1 = (int)(K / 64);
  cfg.S2 = (int)(w.r64 / 64);
  cfg.splits = 1;
  cfg.steps_per_split = cfg.S1 + cfg.S2;
  cfg.epi = EpiBf16{Y, N, M, N};
  cfg.cb = codebook_of(W);
  set_xcd_order(cfg);
  QLORA_TRY(record_if(ev0, stream));
  QLORA_TRY((run<256, 128, LA1, LB1, LA2, LB2, EpiBf16, false>(cfg, stream)));
  return record_if(ev1, stream);
}

namespace {

// dX = dY W' + (second segment) on 256 x 128 tiles: the frozen weight's
// tiles are dequantized and transposed into LDS, the LoRA columns
// (s G | A^T) form the second segment.
template <class Epi>
hipError_t input_grad(const uint16_t* dY, Nf4Weight W, const uint16_t* apad, int64_t M,
                      int64_t N, int64_t K, const WsLayout& w, char* ws, Epi epi,
                      hipStream_t stream) {
  using LA1 = DirectRows<256>;
  using LB1 = Nf4Cols<128>;
  using LA2 = DirectRows<256>;
  using LB2 = DirectRows<128>;
  Contraction<256, 128, LA1, LB1, LA2, LB2, Epi> cfg{};
  cfg.a1 = LA1{dY, N, M};
  cfg.b1 = LB1{W.codes, W.absmax_q, W.absmax_s2, N, K, nf4_consts(W)};
  cfg.a2 = LA2{reinterpret_cast<const uint16_t*>(ws + w.sg), w.r64, M};
  cfg.b2 = LB2{apad, w.r64, K};
  cfg.nP = (int)ceil_div(M, 256);
  cfg.nQ = (int)ceil_div(K, 128);
  cfg.S1 = (int)ceil_div(N, 64);
  cfg.S2 = (int)(w.r64 / 64);
  cfg.splits = 1;
  cfg.steps_per_split = cfg.S1 + cfg.S2;
  cfg.epi = epi;
  cfg.cb = codebook_of(W);
  set_xcd_order(cfg);
  if (Epi::kKeepSeg2 && cfg.S2 > 3) return hipErrorInvalidValue;  // rejected by the API
  return run<256, 128, LA1, LB1, LA2, LB2, Epi, false>(cfg, stream);
}

// dA = X^T (s G) and dB^T = dY^T (s T): both contractions in one launch
// (Aop[k][m] = X[m][k], Aop[n][m] = dY[m][n]; Bop[j][m] = (sG)^T[j][m],
// (sT)^T[j][m]), then the split-order reduce.
template <class LA>
hipError_t adapter_grads(LA xa, LA ya, int64_t M, int64_t N, int64_t K, int r, const WsLayout& w,
                         char* ws, float* dA, float* dB, hipStream_t stream) {
  using LB = DirectRows<64>;
  using C = Contraction<128, 64, LA, LB, LoadNone, LoadNone, EpiPartial>;
  float* part = reinterpret_cast<float*>(ws + w.part);
  const int64_t splits = grad_splits(M, N, K, w.r64);
  const int64_t steps = ceil_div(M, 64);
  float* pa = part;
  float* pb = part + K * w.r64 * splits;
  C ca{}, cb{};
  ca.a1 = xa;
  ca.b1 = LB{reinterpret_cast<const uint16_t*>(ws + w.sgt), w.Mp, w.r64};
  ca.nP = (int)ceil_div(K, 128);
  ca.epi = EpiPartial{pa, K, w.r64};
  cb.a1 = ya;
  cb.b1 = LB{reinterpret_cast<const uint16_t*>(ws + w.stt), w.Mp, w.r64};
  cb.nP = (int)ceil_div(N, 128);
  cb.epi = EpiPartial{pb, N, w.r64};
  for (C* c : {&ca, &cb}) {
    c->nQ = (int)(w.r64 / 64);
    c->S1 = (int)steps;
    c->S2 = 0;
    c->steps_per_split = (int)ceil_div(steps, splits);
    c->splits = (int)ceil_div(steps, c->steps_per_split);
  }
  QLORA_TRY((run_pair<128, 64, LA, LB, LoadNone, LoadNone, EpiPartial, true>(ca, cb, stream)));
  hipLaunchKernelGGL(reduce_grads_kernel, dim3(grid_for((K + N) * (w.r64 / 4))), dim3(256), 0,
                     stream, pa, pb, ca.splits, K, N, r, w.r64, dA, dB);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const uint16_t* dY, const uint16_t* X, const float* T, Nf4Weight W,
                      const uint16_t* A, const uint16_t* B, int64_t M, int64_t N, int64_t K,
                      int r, float scale, uint16_t* dX, float* dA, float* dB, void* ws_,
                      hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1, Dropout dr) {
  char* ws = reinterpret_cast<char*>(ws_);
  const WsLayout w = ws_layout(M, N, K, r);
  float* part = reinterpret_cast<float*>(ws + w.part);
  QLORA_TRY(prep_adapter(A, K, r, w, ws, stream));
  const uint16_t* apad =
      adapter_in_place(A, r) ? A : reinterpret_cast<const uint16_t*>(ws + w.apad);

  // 1. G = dY B^T  (Bop[j][n] = B[j][n], rows j < r), reduced together with
  // 2. bf16 (s T)^T from the caller's T (or T recomputed when there is none)
  {
    int splits = 0;
    DirectRows<64> lb{B, N, (int64_t)r};
    QLORA_TRY(lowrank_partials(DirectRows<64>{dY, N, M}, M, N, lb, w.r64, part, &splits, stream));
    // under dropout, s f G feeds both the masked dX columns and dA
    LowrankJob jg{part, splits, w.r64, nullptr, reinterpret_cast<uint16_t*>(ws + w.sg),
                  reinterpret_cast<uint16_t*>(ws + w.sgt)};
    if (dr.mask) jg.f = dr.keep_scale;
    const LowrankJob jt = T ? LowrankJob{T, 1, (int64_t)r, nullptr, nullptr,
                                         reinterpret_cast<uint16_t*>(ws + w.stt)}
                            : LowrankJob{};
    hipLaunchKernelGGL(reduce_lowrank_kernel, dim3(grid_for((T ? 2 : 1) * w.Mp * w.r64)),
                       dim3(256), 0, stream, jg, jt, M, r, w.r64, w.Mp, scale);
    QLORA_TRY(hipGetLastError());
  }
  if (!T) {
    QLORA_TRY(compute_T(X, A, M, K, r, w, ws, scale, reinterpret_cast<float*>(ws + w.t32),
                        true, dr, stream));
  }
  // 3. dX = dY W' + (s G) A^T   (+ keep o ((s f G) A^T) under dropout)
  if (dX) {
    QLORA_TRY(record_if(ev0, stream));
    if (dr.mask)
      QLORA_TRY(input_grad(dY, W, apad, M, N, K, w, ws, EpiBf16Keep{dX, K, M, K, dr.mask, K / 32},
                           stream));
    else
      QLORA_TRY(input_grad(dY, W, apad, M, N, K, w, ws, EpiBf16{dX, K, M, K}, stream));
    QLORA_TRY(record_if(ev1, stream));
  }
  // 4. dA = X^T (s G) (P = K) and dB^T = dY^T (s T) (P = N): Q = r64,
  //    contraction over M, one launch for both, then one reduce; under
  //    dropout the X operand passes through the keep mask (D(X)^T (s f G))
  if (dr.mask) {
    using LA = ColsBf16<128, true>;
    return adapter_grads(LA{X, K, M, K, dr.mask, K / 32}, LA{dY, N, M, N, nullptr, 0}, M, N, K,
                         r, w, ws, dA, dB, stream);
  }
  return adapter_grads(ColsBf16<128>{X, K, M, K}, ColsBf16<128>{dY, N, M, N}, M, N, K, r, w, ws,
                       dA, dB, stream);
}

// exported for the small-M path, which shares the workspace layout
size_t ws_offset_part(int64_t M, int64_t N, int64_t K, int r) { return ws_layout(M, N, K, r).part; }

}  // namespace qlora
