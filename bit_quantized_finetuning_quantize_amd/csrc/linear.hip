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
//   2. T (recomputed when the caller passes none) and bf16 (s T)^T
//   3. dX = dY W' + (sG) A^T   one contraction over N + r; the weight tile is
//                         dequantized and transposed into LDS
//   4. dA = X^T (sG),  dB = (sT)^T dY   split-M contractions -> reduce
#include "common.h"
#include "gemm.h"
#include "kernels.h"

#include <algorithm>

namespace qlora {

using namespace gemm;

namespace {

constexpr int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }
constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Number of contraction splits for a split-K launch: about two workgroups
// per compute unit, at least two steps per split.
int64_t choose_splits(int64_t tiles, int64_t steps) {
  int64_t want = ceil_div(512, std::max<int64_t>(tiles, 1));
  int64_t maxs = std::max<int64_t>(1, steps / 2);
  int64_t s = std::min(want, maxs);
  if (s < 1) s = 1;
  const int64_t per = ceil_div(steps, s);
  return ceil_div(steps, per);
}

// ---------------------------------------------------------------------------
// workspace carve-up (byte offsets, 256-aligned)
struct WsLayout {
  int64_t r64, Mp;
  size_t apad, at, t32, st, stt, g32, sg, sgt, part, total;
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
  w.g32 = take((size_t)M * r * 4);
  w.sg = take((size_t)w.Mp * w.r64 * 2);
  w.sgt = take((size_t)w.r64 * w.Mp * 2);
  // split-K partials: the largest of the four low-rank contractions
  size_t pe = 0;
  auto consider = [&](int64_t P, int64_t Q, int64_t splits) {
    pe = std::max(pe, (size_t)(P * Q * splits));
  };
  consider(M, w.r64, choose_splits(ceil_div(M, 64) * (w.r64 / 64), ceil_div(K, 64)));
  consider(M, w.r64, choose_splits(ceil_div(M, 64) * (w.r64 / 64), ceil_div(N, 64)));
  consider(K, w.r64, choose_splits(ceil_div(K, 128) * (w.r64 / 64), ceil_div(M, 64)));
  consider(w.r64, N, choose_splits((w.r64 / 64) * ceil_div(N, 128), ceil_div(M, 64)));
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
template __global__ void contraction_kernel<128, 64, ColsBf16<128>, DirectRows<64>, LoadNone,
    LoadNone, EpiPartial, true>(
    Contraction<128, 64, ColsBf16<128>, DirectRows<64>, LoadNone, LoadNone, EpiPartial>);
template __global__ void contraction_kernel<64, 128, DirectRows<64>, ColsBf16<128>, LoadNone,
    LoadNone, EpiPartial, true>(
    Contraction<64, 128, DirectRows<64>, ColsBf16<128>, LoadNone, LoadNone, EpiPartial>);
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
// [split][M][ld]) and emit: float32 V (optional), bf16(s V) padded
// [Mp x r64] and its transpose [r64 x Mp] (optional).
__global__ void reduce_lowrank_kernel(const float* __restrict__ part, int splits,
                                      int64_t ld, int64_t M, int r, int64_t r64,
                                      int64_t Mp, float s, float* __restrict__ out32,
                                      uint16_t* __restrict__ sv,
                                      uint16_t* __restrict__ svt) {
  const int64_t total = Mp * r64;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = i / r64, j = i % r64;
    float v = 0.0f;
    if (m < M && j < r) {
      for (int sp = 0; sp < splits; ++sp) v += part[((int64_t)sp * M + m) * ld + j];
      if (out32) out32[m * r + j] = v;
    }
    const uint16_t b = (uint16_t)(pack_bf16x2(s * v, 0.0f) & 0xffffu);
    sv[i] = b;
    if (svt) svt[j * Mp + m] = b;
  }
}

// out[p][q] = sum_s part[s][p][q] for p < Pv, q < Qv (partials dense P x Q).
__global__ void reduce_plain_kernel(const float* __restrict__ part, int splits, int64_t P,
                                    int64_t Q, int64_t Pv, int64_t Qv,
                                    float* __restrict__ out, int64_t ldo) {
  const int64_t total = Pv * Qv;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t p = i / Qv, q = i % Qv;
    float v = 0.0f;
    for (int sp = 0; sp < splits; ++sp) v += part[((int64_t)sp * P + p) * Q + q];
    out[p * ldo + q] = v;
  }
}

unsigned grid_for(int64_t total, int threads = 256) {
  int64_t b = ceil_div(total, threads);
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(b, 8192));
}

// ---------------------------------------------------------------------------
// launching a contraction

template <int PT, int QT, class LA1, class LB1, class LA2, class LB2, class Epi, bool kPartial>
hipError_t run(Contraction<PT, QT, LA1, LB1, LA2, LB2, Epi> cfg, hipStream_t stream) {
  auto kern = contraction_kernel<PT, QT, LA1, LB1, LA2, LB2, Epi, kPartial>;
  const size_t lds = lds_bytes<PT, QT>();
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int64_t blocks = (int64_t)cfg.nP * cfg.nQ * cfg.splits;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(threads_for<PT, LB1>()), lds, stream, cfg);
  return hipGetLastError();
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
// Aop rows come from a bf16 row-major source (ld lda, contraction length C).
template <class LB>
hipError_t lowrank_partials(const uint16_t* a, int64_t lda, int64_t M, int64_t C, LB lb,
                            int64_t r64, float* part, int* splits_out, hipStream_t stream) {
  using LA = DirectRows<64>;
  Contraction<64, 64, LA, LB, LoadNone, LoadNone, EpiPartial> cfg{};
  cfg.a1 = LA{a, lda, M};
  cfg.b1 = lb;
  cfg.nP = (int)ceil_div(M, 64);
  cfg.nQ = (int)(r64 / 64);
  set_steps(cfg, ceil_div(C, 64), 0, (int64_t)cfg.nP * cfg.nQ);
  cfg.epi = EpiPartial{part, M, r64};
  *splits_out = cfg.splits;
  return run<64, 64, LA, LB, LoadNone, LoadNone, EpiPartial, true>(cfg, stream);
}

#define QLORA_TRY(x)                       \
  do {                                     \
    hipError_t e_ = (x);                   \
    if (e_ != hipSuccess) return e_;       \
  } while (0)

hipError_t prep_adapter(const uint16_t* A, int64_t K, int r, const WsLayout& w, char* ws,
                        hipStream_t stream) {
  hipLaunchKernelGGL(adapter_prep_kernel, dim3(grid_for(K * w.r64)), dim3(256), 0, stream, A, K,
                     r, w.r64, reinterpret_cast<uint16_t*>(ws + w.apad),
                     reinterpret_cast<uint16_t*>(ws + w.at));
  return hipGetLastError();
}

// T = X A -> out32 (optional), bf16(s T) [Mp x r64], bf16(s T)^T (optional).
hipError_t compute_T(const uint16_t* X, const uint16_t* At, int64_t M, int64_t K, int r,
                     const WsLayout& w, char* ws, float s, float* out32, bool transposed,
                     hipStream_t stream) {
  float* part = reinterpret_cast<float*>(ws + w.part);
  int splits = 0;
  // Bop[j][k] = A^T[j][k]: rows of the transposed, padded adapter
  DirectRows<64> lb{At, K, w.r64};
  QLORA_TRY(lowrank_partials(X, K, M, K, lb, w.r64, part, &splits, stream));
  hipLaunchKernelGGL(reduce_lowrank_kernel, dim3(grid_for(w.Mp * w.r64)), dim3(256), 0, stream,
                     part, splits, w.r64, M, r, w.r64, w.Mp, s, out32,
                     reinterpret_cast<uint16_t*>(ws + w.st),
                     transposed ? reinterpret_cast<uint16_t*>(ws + w.stt) : nullptr);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_gemm(const uint16_t* X, Nf4Weight W, const uint16_t* A,
                           const uint16_t* B, int64_t M, int64_t N, int64_t K, int r,
                           float scale, uint16_t* Y, float* T_out, void* ws_,
                           hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  char* ws = reinterpret_cast<char*>(ws_);
  const WsLayout w = ws_layout(M, N, K, r);
  QLORA_TRY(prep_adapter(A, K, r, w, ws, stream));
  const uint16_t* at = reinterpret_cast<const uint16_t*>(ws + w.at);
  float* t32 = T_out ? T_out : reinterpret_cast<float*>(ws + w.t32);
  QLORA_TRY(compute_T(X, at, M, K, r, w, ws, scale, t32, false, stream));

  using LA1 = DirectRows<256>;
  using LB1 = Nf4Rows<128>;
  using LA2 = DirectRows<256>;
  using LB2 = ColsBf16<128>;
  Contraction<256, 128, LA1, LB1, LA2, LB2, EpiBf16> cfg{};
  cfg.a1 = LA1{X, K, M};
  cfg.b1 = LB1{W.codes, W.absmax_q, W.absmax_s2, N, K};
  cfg.a2 = LA2{reinterpret_cast<const uint16_t*>(ws + w.st), w.r64, M};
  cfg.b2 = LB2{B, N, (int64_t)r, N};  // Bop[n][j] = B[j][n]
  cfg.nP = (int)ceil_div(M, 256);
  cfg.nQ = (int)ceil_div(N, 128);
  cfg.S1 = (int)(K / 64);
  cfg.S2 = (int)(w.r64 / 64);
  cfg.splits = 1;
  cfg.steps_per_split = cfg.S1 + cfg.S2;
  cfg.epi = EpiBf16{Y, N, M, N};
  QLORA_TRY(record_if(ev0, stream));
  QLORA_TRY((run<256, 128, LA1, LB1, LA2, LB2, EpiBf16, false>(cfg, stream)));
  return record_if(ev1, stream);
}

hipError_t launch_bwd(const uint16_t* dY, const uint16_t* X, const float* T, Nf4Weight W,
                      const uint16_t* A, const uint16_t* B, int64_t M, int64_t N, int64_t K,
                      int r, float scale, uint16_t* dX, float* dA, float* dB, void* ws_,
                      hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  char* ws = reinterpret_cast<char*>(ws_);
  const WsLayout w = ws_layout(M, N, K, r);
  float* part = reinterpret_cast<float*>(ws + w.part);
  QLORA_TRY(prep_adapter(A, K, r, w, ws, stream));
  const uint16_t* apad = reinterpret_cast<const uint16_t*>(ws + w.apad);
  const uint16_t* at = reinterpret_cast<const uint16_t*>(ws + w.at);

  // 1. G = dY B^T  (Bop[j][n] = B[j][n], rows j < r)
  {
    int splits = 0;
    DirectRows<64> lb{B, N, (int64_t)r};
    QLORA_TRY(lowrank_partials(dY, N, M, N, lb, w.r64, part, &splits, stream));
    hipLaunchKernelGGL(reduce_lowrank_kernel, dim3(grid_for(w.Mp * w.r64)), dim3(256), 0, stream,
                       part, splits, w.r64, M, r, w.r64, w.Mp, scale,
                       reinterpret_cast<float*>(ws + w.g32),
                       reinterpret_cast<uint16_t*>(ws + w.sg),
                       reinterpret_cast<uint16_t*>(ws + w.sgt));
    QLORA_TRY(hipGetLastError());
  }
  // 2. bf16 (s T)^T, recomputing T if needed
  if (T) {
    hipLaunchKernelGGL(reduce_lowrank_kernel, dim3(grid_for(w.Mp * w.r64)), dim3(256), 0, stream,
                       T, 1, (int64_t)r, M, r, w.r64, w.Mp, scale, (float*)nullptr,
                       reinterpret_cast<uint16_t*>(ws + w.st),
                       reinterpret_cast<uint16_t*>(ws + w.stt));
    QLORA_TRY(hipGetLastError());
  } else {
    QLORA_TRY(compute_T(X, at, M, K, r, w, ws, scale, reinterpret_cast<float*>(ws + w.t32),
                        true, stream));
  }
  // 3. dX = dY W' + (s G) A^T
  if (dX) {
    using LA1 = DirectRows<256>;
    using LB1 = Nf4Cols<128>;
    using LA2 = DirectRows<256>;
    using LB2 = DirectRows<128>;
    Contraction<256, 128, LA1, LB1, LA2, LB2, EpiBf16> cfg{};
    cfg.a1 = LA1{dY, N, M};
    cfg.b1 = LB1{W.codes, W.absmax_q, W.absmax_s2, N, K};
    cfg.a2 = LA2{reinterpret_cast<const uint16_t*>(ws + w.sg), w.r64, M};
    cfg.b2 = LB2{apad, w.r64, K};
    cfg.nP = (int)ceil_div(M, 256);
    cfg.nQ = (int)ceil_div(K, 128);
    cfg.S1 = (int)ceil_div(N, 64);
    cfg.S2 = (int)(w.r64 / 64);
    cfg.splits = 1;
    cfg.steps_per_split = cfg.S1 + cfg.S2;
    cfg.epi = EpiBf16{dX, K, M, K};
    QLORA_TRY(record_if(ev0, stream));
    QLORA_TRY((run<256, 128, LA1, LB1, LA2, LB2, EpiBf16, false>(cfg, stream)));
    QLORA_TRY(record_if(ev1, stream));
  }
  // 4a. dA = X^T (s G): P = K, Q = r64, contraction over M
  {
    using LA = ColsBf16<128>;    // Aop[k][m] = X[m][k]
    using LB = DirectRows<64>;   // Bop[j][m] = (sG)^T[j][m]
    Contraction<128, 64, LA, LB, LoadNone, LoadNone, EpiPartial> cfg{};
    cfg.a1 = LA{X, K, M, K};
    cfg.b1 = LB{reinterpret_cast<const uint16_t*>(ws + w.sgt), w.Mp, w.r64};
    cfg.nP = (int)ceil_div(K, 128);
    cfg.nQ = (int)(w.r64 / 64);
    set_steps(cfg, ceil_div(M, 64), 0, (int64_t)cfg.nP * cfg.nQ);
    cfg.epi = EpiPartial{part, K, w.r64};
    QLORA_TRY((run<128, 64, LA, LB, LoadNone, LoadNone, EpiPartial, true>(cfg, stream)));
    hipLaunchKernelGGL(reduce_plain_kernel, dim3(grid_for(K * r)), dim3(256), 0, stream, part,
                       cfg.splits, K, w.r64, K, (int64_t)r, dA, (int64_t)r);
    QLORA_TRY(hipGetLastError());
  }
  // 4b. dB = (s T)^T dY: P = r64, Q = N, contraction over M
  {
    using LA = DirectRows<64>;   // Aop[j][m] = (sT)^T[j][m]
    using LB = ColsBf16<128>;    // Bop[n][m] = dY[m][n]
    Contraction<64, 128, LA, LB, LoadNone, LoadNone, EpiPartial> cfg{};
    cfg.a1 = LA{reinterpret_cast<const uint16_t*>(ws + w.stt), w.Mp, w.r64};
    cfg.b1 = LB{dY, N, M, N};
    cfg.nP = (int)(w.r64 / 64);
    cfg.nQ = (int)ceil_div(N, 128);
    set_steps(cfg, ceil_div(M, 64), 0, (int64_t)cfg.nP * cfg.nQ);
    cfg.epi = EpiPartial{part, w.r64, N};
    QLORA_TRY((run<64, 128, LA, LB, LoadNone, LoadNone, EpiPartial, true>(cfg, stream)));
    hipLaunchKernelGGL(reduce_plain_kernel, dim3(grid_for((int64_t)r * N)), dim3(256), 0, stream,
                       part, cfg.splits, w.r64, N, (int64_t)r, N, dB, N);
    QLORA_TRY(hipGetLastError());
  }
  return hipSuccess;
}

// exported for the small-M path, which shares the workspace layout
size_t ws_offset_part(int64_t M, int64_t N, int64_t K, int r) { return ws_layout(M, N, K, r).part; }

}  // namespace qlora
