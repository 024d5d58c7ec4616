// C ABI of the library: argument validation, dispatch, status codes.
// Every check runs before anything is enqueued; a rejected call has no side
// effects and makes no HIP call.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/qlora.h"
#include "common.h"
#include "kernels.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return QLORA_OK;
  g_last_hip_error = (int)e;
  return QLORA_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr int64_t kMaxGroups = 0x7fffffffLL;  // grid limit of the quantize launch

// absmax_q may be null: a store without double quantization
int check_store(const uint8_t* codes, const uint8_t* absmax_q, const float* absmax_s2) {
  (void)absmax_q;
  if (!codes || !absmax_s2) return QLORA_ERR_INVALID_ARG;
  if (!aligned(codes, 16) || !aligned(absmax_s2, 4)) return QLORA_ERR_UNSUPPORTED;
  return QLORA_OK;
}

bool valid_store_type(int32_t t) { return t >= 0 && t <= (QLORA_STORE_FP4 | QLORA_STORE_DQ_FP8); }

int check_linear_shape(int64_t M, int64_t N, int64_t K, int32_t r) {
  if (M <= 0 || N <= 0 || K <= 0) return QLORA_ERR_INVALID_ARG;
  if (K % QLORA_NF4_BLOCK != 0 || N % QLORA_NF4_BLOCK != 0) return QLORA_ERR_UNSUPPORTED;
  if (r < 1 || r > QLORA_MAX_RANK) return QLORA_ERR_UNSUPPORTED;
  if (M > (int64_t)1 << 30 || N > (int64_t)1 << 30 || K > (int64_t)1 << 30) return QLORA_ERR_UNSUPPORTED;
  // The kernels address their operands with 32-bit buffer offsets: every
  // bf16 activation matrix stays below 2^30 elements (2 GiB), the NF4 codes
  // below 2 GiB, and a row below 2^21 elements (a 256-row tile spans at most
  // 1 GiB).
  if (N > (int64_t)1 << 21 || K > (int64_t)1 << 21) return QLORA_ERR_UNSUPPORTED;
  if (M * N >= (int64_t)1 << 30 || M * K >= (int64_t)1 << 30 || N * K >= (int64_t)1 << 32)
    return QLORA_ERR_UNSUPPORTED;
  return QLORA_OK;
}

// 16-bit keep threshold of a drop probability p in [0, 1): floor(p 2^16 + 1/2)
// (p * 2^16 is exact in double). Returns -1 for p outside [0, 1) or NaN, and
// 65536 when p rounds to certain dropping.
int64_t keep_threshold(float p) {
  if (!(p >= 0.0f && p < 1.0f)) return -1;
  return (int64_t)std::floor((double)p * 65536.0 + 0.5);
}

int check_dropout(const uint32_t* mask, float p, qlora::Dropout* dr) {
  if (!mask) return QLORA_ERR_INVALID_ARG;
  const int64_t thr = keep_threshold(p);
  if (thr < 0) return QLORA_ERR_INVALID_ARG;
  if (thr >= 65536) return QLORA_ERR_UNSUPPORTED;
  if (!aligned(mask, 4)) return QLORA_ERR_UNSUPPORTED;
  dr->mask = mask;
  dr->keep_scale = (float)(65536.0 / (double)(65536 - thr));
  return QLORA_OK;
}

}  // namespace

extern "C" {

int64_t qlora_nf4_codes_bytes(int64_t numel) { return numel < 0 ? -1 : (numel + 1) / 2; }
int64_t qlora_nf4_num_blocks(int64_t numel) {
  return numel < 0 ? -1 : (numel + QLORA_NF4_BLOCK - 1) / QLORA_NF4_BLOCK;
}
int64_t qlora_nf4_num_groups(int64_t numel) {
  return numel < 0 ? -1 : (qlora_nf4_num_blocks(numel) + QLORA_NF4_GROUP - 1) / QLORA_NF4_GROUP;
}

void qlora_nf4_codebook(float* levels) {
  if (!levels) return;
  std::memcpy(levels, qlora::kNF4, sizeof(qlora::kNF4));
}

int qlora_nf4_quantize_ex(const uint16_t* w, int64_t numel, uint8_t* codes, uint8_t* absmax_q,
                          float* absmax_s2, int32_t store_type, void* stream) {
  if (!w || numel <= 0) return QLORA_ERR_INVALID_ARG;
  if (!codes || !absmax_s2) return QLORA_ERR_INVALID_ARG;  // absmax_q null: no DQ
  if (!valid_store_type(store_type)) return QLORA_ERR_INVALID_ARG;
  if (!aligned(w, 2) || !aligned(codes, 4) || !aligned(absmax_s2, 4)) return QLORA_ERR_UNSUPPORTED;
  if (qlora_nf4_num_groups(numel) > kMaxGroups) return QLORA_ERR_UNSUPPORTED;
  return hip_status(qlora::launch_nf4_quantize(w, numel, codes, absmax_q, absmax_s2, store_type,
                                               reinterpret_cast<hipStream_t>(stream)));
}

int qlora_nf4_quantize(const uint16_t* w, int64_t numel, uint8_t* codes, uint8_t* absmax_q,
                       float* absmax_s2, void* stream) {
  return qlora_nf4_quantize_ex(w, numel, codes, absmax_q, absmax_s2, QLORA_STORE_NF4, stream);
}

static int dequant_common(const uint8_t* codes, const uint8_t* absmax_q, const float* absmax_s2,
                          int64_t numel, int32_t store_type, void* out, bool bf16, void* stream) {
  if (!codes || !absmax_s2 || !out || numel <= 0) return QLORA_ERR_INVALID_ARG;
  if (!valid_store_type(store_type)) return QLORA_ERR_INVALID_ARG;
  if (!aligned(codes, 4) || !aligned(absmax_s2, 4) || !aligned(out, 16)) return QLORA_ERR_UNSUPPORTED;
  return hip_status(qlora::launch_nf4_dequantize(qlora::Nf4Weight{codes, absmax_q, absmax_s2,
                                                                  store_type},
                                                 numel, out, bf16,
                                                 reinterpret_cast<hipStream_t>(stream)));
}

int qlora_nf4_dequantize_ex(const uint8_t* codes, const uint8_t* absmax_q,
                            const float* absmax_s2, int64_t numel, int32_t store_type,
                            float* out, void* stream) {
  return dequant_common(codes, absmax_q, absmax_s2, numel, store_type, out, false, stream);
}

int qlora_nf4_dequantize_bf16_ex(const uint8_t* codes, const uint8_t* absmax_q,
                                 const float* absmax_s2, int64_t numel, int32_t store_type,
                                 uint16_t* out, void* stream) {
  return dequant_common(codes, absmax_q, absmax_s2, numel, store_type, out, true, stream);
}

int qlora_nf4_dequantize(const uint8_t* codes, const uint8_t* absmax_q, const float* absmax_s2,
                         int64_t numel, float* out, void* stream) {
  return dequant_common(codes, absmax_q, absmax_s2, numel, QLORA_STORE_NF4, out, false, stream);
}

int qlora_nf4_dequantize_bf16(const uint8_t* codes, const uint8_t* absmax_q,
                              const float* absmax_s2, int64_t numel, uint16_t* out,
                              void* stream) {
  return dequant_common(codes, absmax_q, absmax_s2, numel, QLORA_STORE_NF4, out, true, stream);
}

int qlora_nf4_merge(const uint8_t* codes, const uint8_t* absmax_q, const float* absmax_s2,
                    int64_t N, int64_t K, const uint16_t* A, const uint16_t* B, int32_t r,
                    float scale, uint16_t* out, void* stream) {
  return qlora_nf4_merge_ex(codes, absmax_q, absmax_s2, N, K, A, B, r, scale, QLORA_STORE_NF4,
                            out, stream);
}

int qlora_nf4_merge_ex(const uint8_t* codes, const uint8_t* absmax_q, const float* absmax_s2,
                       int64_t N, int64_t K, const uint16_t* A, const uint16_t* B, int32_t r,
                       float scale, int32_t store_type, uint16_t* out, void* stream) {
  if (!A || !B || !out) return QLORA_ERR_INVALID_ARG;
  if (!valid_store_type(store_type)) return QLORA_ERR_INVALID_ARG;
  int st = check_store(codes, absmax_q, absmax_s2);
  if (st != QLORA_OK) return st;
  if (N <= 0 || K <= 0) return QLORA_ERR_INVALID_ARG;
  if (K % QLORA_NF4_BLOCK != 0 || r < 1 || r > QLORA_MAX_RANK) return QLORA_ERR_UNSUPPORTED;
  if (N > (int64_t)1 << 30 || K > (int64_t)1 << 30 || (N + 63) / 64 > 65535)
    return QLORA_ERR_UNSUPPORTED;
  if (!aligned(A, 2) || !aligned(B, 2) || !aligned(out, 16)) return QLORA_ERR_UNSUPPORTED;
  return hip_status(qlora::launch_nf4_merge(qlora::Nf4Weight{codes, absmax_q, absmax_s2, store_type},
                                            N, K, A, B, r, scale, out,
                                            reinterpret_cast<hipStream_t>(stream)));
}

int qlora_adamw_step(float* p, float* m, float* v, const float* g, int64_t n, float lr,
                     float beta1, float beta2, float eps, float weight_decay, int64_t step,
                     uint16_t* p_bf16, void* stream) {
  if (!p || !m || !v || !g || n <= 0 || step < 1) return QLORA_ERR_INVALID_ARG;
  if (!(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f) || !(eps > 0.0f))
    return QLORA_ERR_INVALID_ARG;
  if (!aligned(p, 4) || !aligned(m, 4) || !aligned(v, 4) || !aligned(g, 4) ||
      (p_bf16 && !aligned(p_bf16, 2)))
    return QLORA_ERR_UNSUPPORTED;
  return hip_status(qlora::launch_adamw(p, m, v, g, n, lr, beta1, beta2, eps, weight_decay, step,
                                        p_bf16, reinterpret_cast<hipStream_t>(stream)));
}

int qlora_adamw8_step(float* p, uint8_t* m8, float* m_scale, uint8_t* v8, float* v_scale,
                      const float* g, int64_t n, float lr, float beta1, float beta2, float eps,
                      float weight_decay, int64_t step, uint16_t* p_bf16, void* stream) {
  if (!p || !m8 || !m_scale || !v8 || !v_scale || !g || n <= 0 || step < 1)
    return QLORA_ERR_INVALID_ARG;
  if (!(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f) || !(eps > 0.0f))
    return QLORA_ERR_INVALID_ARG;
  if (!aligned(p, 4) || !aligned(g, 4) || !aligned(m_scale, 4) || !aligned(v_scale, 4) ||
      (p_bf16 && !aligned(p_bf16, 2)))
    return QLORA_ERR_UNSUPPORTED;
  return hip_status(qlora::launch_adamw8(p, m8, m_scale, v8, v_scale, g, n, lr, beta1, beta2, eps,
                                         weight_decay, step, p_bf16,
                                         reinterpret_cast<hipStream_t>(stream)));
}

size_t qlora_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t r) {
  if (check_linear_shape(M, N, K, r) != QLORA_OK) return 0;
  return qlora::linear_workspace_bytes(M, N, K, r);
}

static int linear_fwd_impl(const uint16_t* X, const uint8_t* codes, const uint8_t* absmax_q,
                           const float* absmax_s2, const uint16_t* A, const uint16_t* B,
                           int64_t M, int64_t N, int64_t K, int32_t r, float scale, uint16_t* Y,
                           float* T_out, void* ws, size_t ws_bytes, int32_t store_type,
                           void* stream, void* ev_begin, void* ev_end) {
  if (!X || !A || !B || !Y) return QLORA_ERR_INVALID_ARG;
  if (!valid_store_type(store_type)) return QLORA_ERR_INVALID_ARG;
  int st = check_store(codes, absmax_q, absmax_s2);
  if (st != QLORA_OK) return st;
  st = check_linear_shape(M, N, K, r);
  if (st != QLORA_OK) return st;
  if (!aligned(X, 16) || !aligned(B, 16) || !aligned(A, 2) || !aligned(Y, 2) ||
      (T_out && !aligned(T_out, 4)))
    return QLORA_ERR_UNSUPPORTED;
  const size_t need = qlora::linear_workspace_bytes(M, N, K, r);
  if (!ws || ws_bytes < need) return QLORA_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return QLORA_ERR_UNSUPPORTED;
  qlora::Nf4Weight W{codes, absmax_q, absmax_s2, store_type};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipEvent_t e0 = reinterpret_cast<hipEvent_t>(ev_begin);
  hipEvent_t e1 = reinterpret_cast<hipEvent_t>(ev_end);
  if (M <= qlora::kGemvMaxM)
    return hip_status(
        qlora::launch_fwd_gemv(X, W, A, B, (int)M, N, K, r, scale, Y, T_out, ws, s, e0, e1));
  return hip_status(qlora::launch_fwd_gemm(X, W, A, B, M, N, K, r, scale, Y, T_out, ws, s, e0, e1));
}

int qlora_linear_fwd_profiled(const uint16_t* X, const uint8_t* codes, const uint8_t* absmax_q,
                              const float* absmax_s2, const uint16_t* A, const uint16_t* B,
                              int64_t M, int64_t N, int64_t K, int32_t r, float scale,
                              uint16_t* Y, float* T_out, void* ws, size_t ws_bytes, void* stream,
                              void* ev_begin, void* ev_end) {
  return linear_fwd_impl(X, codes, absmax_q, absmax_s2, A, B, M, N, K, r, scale, Y, T_out, ws,
                         ws_bytes, QLORA_STORE_NF4, stream, ev_begin, ev_end);
}

int qlora_linear_fwd(const uint16_t* X, const uint8_t* codes, const uint8_t* absmax_q,
                     const float* absmax_s2, const uint16_t* A, const uint16_t* B, int64_t M,
                     int64_t N, int64_t K, int32_t r, float scale, uint16_t* Y, float* T_out,
                     void* ws, size_t ws_bytes, void* stream) {
  return linear_fwd_impl(X, codes, absmax_q, absmax_s2, A, B, M, N, K, r, scale, Y, T_out, ws,
                         ws_bytes, QLORA_STORE_NF4, stream, nullptr, nullptr);
}

int qlora_linear_fwd_ex(const uint16_t* X, const uint8_t* codes, const uint8_t* absmax_q,
                        const float* absmax_s2, const uint16_t* A, const uint16_t* B, int64_t M,
                        int64_t N, int64_t K, int32_t r, float scale, uint16_t* Y, float* T_out,
                        void* ws, size_t ws_bytes, int32_t store_type, void* stream) {
  return linear_fwd_impl(X, codes, absmax_q, absmax_s2, A, B, M, N, K, r, scale, Y, T_out, ws,
                         ws_bytes, store_type, stream, nullptr, nullptr);
}

int qlora_linear_fwd_noalloc(const uint16_t* X, const uint8_t* codes, const uint8_t* absmax_q,
                             const float* absmax_s2, const uint16_t* A, const uint16_t* B,
                             int64_t M, int64_t N, int64_t K, int32_t r, float scale, uint16_t* Y,
                             float* T_out, void* stream) {
  static_assert(QLORA_NOALLOC_SCRATCH_BYTES == qlora::kNoAllocScratchBytes, "scratch size");
  if (!X || !A || !B || !Y) return QLORA_ERR_INVALID_ARG;
  int st = check_store(codes, absmax_q, absmax_s2);
  if (st != QLORA_OK) return st;
  st = check_linear_shape(M, N, K, r);
  if (st != QLORA_OK) return st;
  if (!aligned(X, 16) || !aligned(B, 16) || !aligned(A, 2) || !aligned(Y, 2) ||
      (T_out && !aligned(T_out, 4)))
    return QLORA_ERR_UNSUPPORTED;
  if (qlora::linear_workspace_bytes(M, N, K, r) > qlora::kNoAllocScratchBytes)
    return QLORA_ERR_WORKSPACE;
  qlora::Nf4Weight W{codes, absmax_q, absmax_s2};
  return hip_status(qlora::launch_fwd_noalloc(X, W, A, B, M, N, K, r, scale, Y, T_out,
                                              reinterpret_cast<hipStream_t>(stream)));
}

static int linear_bwd_impl(const uint16_t* dY, const uint16_t* X, const float* T,
                           const uint8_t* codes, const uint8_t* absmax_q, const float* absmax_s2,
                           const uint16_t* A, const uint16_t* B, int64_t M, int64_t N, int64_t K,
                           int32_t r, float scale, uint16_t* dX, float* dA, float* dB, void* ws,
                           size_t ws_bytes, int32_t store_type, void* stream, void* ev_begin,
                           void* ev_end) {
  if (!dY || !X || !A || !B || !dA || !dB) return QLORA_ERR_INVALID_ARG;
  if (!valid_store_type(store_type)) return QLORA_ERR_INVALID_ARG;
  int st = check_store(codes, absmax_q, absmax_s2);
  if (st != QLORA_OK) return st;
  st = check_linear_shape(M, N, K, r);
  if (st != QLORA_OK) return st;
  if (!aligned(dY, 16) || !aligned(X, 16) || !aligned(B, 16) || !aligned(A, 2) ||
      (T && !aligned(T, 4)) || (dX && !aligned(dX, 2)) || !aligned(dA, 4) || !aligned(dB, 4))
    return QLORA_ERR_UNSUPPORTED;
  const size_t need = qlora::linear_workspace_bytes(M, N, K, r);
  if (!ws || ws_bytes < need) return QLORA_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return QLORA_ERR_UNSUPPORTED;
  qlora::Nf4Weight W{codes, absmax_q, absmax_s2, store_type};
  return hip_status(qlora::launch_bwd(dY, X, T, W, A, B, M, N, K, r, scale, dX, dA, dB, ws,
                                      reinterpret_cast<hipStream_t>(stream),
                                      reinterpret_cast<hipEvent_t>(ev_begin),
                                      reinterpret_cast<hipEvent_t>(ev_end)));
}

int qlora_linear_bwd_profiled(const uint16_t* dY, const uint16_t* X, const float* T,
                              const uint8_t* codes, const uint8_t* absmax_q,
                              const float* absmax_s2, const uint16_t* A, const uint16_t* B,
                              int64_t M, int64_t N, int64_t K, int32_t r, float scale,
                              uint16_t* dX, float* dA, float* dB, void* ws, size_t ws_bytes,
                              void* stream, void* ev_begin, void* ev_end) {
  return linear_bwd_impl(dY, X, T, codes, absmax_q, absmax_s2, A, B, M, N, K, r, scale, dX, dA,
                         dB, ws, ws_bytes, QLORA_STORE_NF4, stream, ev_begin, ev_end);
}

int qlora_linear_bwd(const uint16_t* dY, const uint16_t* X, const float* T, const uint8_t* codes,
                     const uint8_t* absmax_q, const float* absmax_s2, const uint16_t* A,
                     const uint16_t* B, int64_t M, int64_t N, int64_t K, int32_t r, float scale,
                     uint16_t* dX, float* dA, float* dB, void* ws, size_t ws_bytes,
                     void* stream) {
  return linear_bwd_impl(dY, X, T, codes, absmax_q, absmax_s2, A, B, M, N, K, r, scale, dX, dA,
                         dB, ws, ws_bytes, QLORA_STORE_NF4, stream, nullptr, nullptr);
}

int qlora_linear_bwd_ex(const uint16_t* dY, const uint16_t* X, const float* T,
                        const uint8_t* codes, const uint8_t* absmax_q, const float* absmax_s2,
                        const uint16_t* A, const uint16_t* B, int64_t M, int64_t N, int64_t K,
                        int32_t r, float scale, uint16_t* dX, float* dA, float* dB, void* ws,
                        size_t ws_bytes, int32_t store_type, void* stream) {
  return linear_bwd_impl(dY, X, T, codes, absmax_q, absmax_s2, A, B, M, N, K, r, scale, dX, dA,
                         dB, ws, ws_bytes, store_type, stream, nullptr, nullptr);
}

int qlora_dropout_mask(int64_t M, int64_t K, float p, uint64_t seed, uint64_t offset,
                       uint32_t* mask, void* stream) {
  if (!mask || M <= 0 || K <= 0) return QLORA_ERR_INVALID_ARG;
  const int64_t thr = keep_threshold(p);
  if (thr < 0) return QLORA_ERR_INVALID_ARG;
  if (thr >= 65536 || K % 32 != 0 || !aligned(mask, 4)) return QLORA_ERR_UNSUPPORTED;
  if (M > ((int64_t)1 << 40) / K) return QLORA_ERR_UNSUPPORTED;
  return hip_status(qlora::launch_dropout_mask(M, K, (uint32_t)thr, seed, offset, mask,
                                               reinterpret_cast<hipStream_t>(stream)));
}

int qlora_linear_fwd_dropout(const uint16_t* X, const uint8_t* codes, const uint8_t* absmax_q,
                             const float* absmax_s2, const uint16_t* A, const uint16_t* B,
                             int64_t M, int64_t N, int64_t K, int32_t r, float scale,
                             const uint32_t* keep_mask, float p, uint16_t* Y, float* T_out,
                             void* ws, size_t ws_bytes, void* stream) {
  if (!X || !A || !B || !Y) return QLORA_ERR_INVALID_ARG;
  int st = check_store(codes, absmax_q, absmax_s2);
  if (st != QLORA_OK) return st;
  st = check_linear_shape(M, N, K, r);
  if (st != QLORA_OK) return st;
  qlora::Dropout dr;
  st = check_dropout(keep_mask, p, &dr);
  if (st != QLORA_OK) return st;
  if (!aligned(X, 16) || !aligned(B, 16) || !aligned(A, 2) || !aligned(Y, 2) ||
      (T_out && !aligned(T_out, 4)))
    return QLORA_ERR_UNSUPPORTED;
  const size_t need = qlora::linear_workspace_bytes(M, N, K, r);
  if (!ws || ws_bytes < need) return QLORA_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return QLORA_ERR_UNSUPPORTED;
  qlora::Nf4Weight W{codes, absmax_q, absmax_s2};
  // every M takes the MFMA path: the keep mask enters the X A contraction
  return hip_status(qlora::launch_fwd_gemm(X, W, A, B, M, N, K, r, scale, Y, T_out, ws,
                                           reinterpret_cast<hipStream_t>(stream), nullptr,
                                           nullptr, dr));
}

int qlora_linear_bwd_dropout(const uint16_t* dY, const uint16_t* X, const float* T,
                             const uint8_t* codes, const uint8_t* absmax_q,
                             const float* absmax_s2, const uint16_t* A, const uint16_t* B,
                             int64_t M, int64_t N, int64_t K, int32_t r, float scale,
                             const uint32_t* keep_mask, float p, uint16_t* dX, float* dA,
                             float* dB, void* ws, size_t ws_bytes, void* stream) {
  if (!dY || !X || !A || !B || !dA || !dB) return QLORA_ERR_INVALID_ARG;
  int st = check_store(codes, absmax_q, absmax_s2);
  if (st != QLORA_OK) return st;
  st = check_linear_shape(M, N, K, r);
  if (st != QLORA_OK) return st;
  qlora::Dropout dr;
  st = check_dropout(keep_mask, p, &dr);
  if (st != QLORA_OK) return st;
  if (dX && r > QLORA_MAX_DROPOUT_RANK) return QLORA_ERR_UNSUPPORTED;
  if (!aligned(dY, 16) || !aligned(X, 16) || !aligned(B, 16) || !aligned(A, 2) ||
      (T && !aligned(T, 4)) || (dX && !aligned(dX, 2)) || !aligned(dA, 4) || !aligned(dB, 4))
    return QLORA_ERR_UNSUPPORTED;
  const size_t need = qlora::linear_workspace_bytes(M, N, K, r);
  if (!ws || ws_bytes < need) return QLORA_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return QLORA_ERR_UNSUPPORTED;
  qlora::Nf4Weight W{codes, absmax_q, absmax_s2};
  return hip_status(qlora::launch_bwd(dY, X, T, W, A, B, M, N, K, r, scale, dX, dA, dB, ws,
                                      reinterpret_cast<hipStream_t>(stream), nullptr, nullptr,
                                      dr));
}

int qlora_gemv_wait_limit(int64_t microseconds) {
  if (microseconds < 0 || microseconds > 1000000) return QLORA_ERR_INVALID_ARG;
  qlora::set_gemv_wait_us(microseconds);
  return QLORA_OK;
}

const char* qlora_status_string(int status) {
  switch (status) {
    case QLORA_OK: return "ok";
    case QLORA_ERR_INVALID_ARG: return "invalid argument";
    case QLORA_ERR_UNSUPPORTED: return "unsupported shape, rank or alignment";
    case QLORA_ERR_WORKSPACE: return "workspace missing or too small";
    case QLORA_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int qlora_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
