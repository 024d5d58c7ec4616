// Internal launch interface between the C ABI (api.cpp) and the kernels.
// Launchers enqueue on `stream`, never synchronize, and return the launch
// status. Shapes have been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace qlora {

struct Nf4Weight {
  const uint8_t* codes;
  const uint8_t* absmax_q;
  const float* absmax_s2;
  int store_type = 0;  // kStoreFP4 | kStoreDqFp8 (common.h); 0 is NF4, linear code
};

// The level table and constant code the kernels use for a store. A store
// without double quantization keeps float32 constants, so the constant code
// does not apply (the loaders read it with the 8-bit code forced to 255,
// whose linear value is exactly 1).
inline Codebook codebook_of(const Nf4Weight& W) {
  return make_codebook(W.absmax_q ? W.store_type : (W.store_type & kStoreFP4));
}

hipError_t launch_nf4_quantize(const uint16_t* w, int64_t numel, uint8_t* codes,
                               uint8_t* absmax_q, float* absmax_s2, int store_type,
                               hipStream_t stream);

hipError_t launch_nf4_dequantize(Nf4Weight W, int64_t numel, void* out, bool bf16,
                                 hipStream_t stream);

// Merged 16-bit weight: bf16(w' + s (A B)^T), [N x K] row-major.
hipError_t launch_nf4_merge(Nf4Weight W, int64_t N, int64_t K, const uint16_t* A,
                            const uint16_t* B, int r, float scale, uint16_t* out,
                            hipStream_t stream);

// One AdamW step over n float32 parameters with float32 moments (in place);
// p16 (optional) receives bf16(p).
hipError_t launch_adamw(float* p, float* m, float* v, const float* g, int64_t n, float lr,
                        float beta1, float beta2, float eps, float weight_decay, int64_t step,
                        uint16_t* p16, hipStream_t stream);

// The same step with 8-bit moments: per block of 256 parameters, E4M3 codes
// of m with scale sm[b] and E5M2 codes of v with scale sv[b] (updated in
// place).
hipError_t launch_adamw8(float* p, uint8_t* m8, float* sm, uint8_t* v8, float* sv, const float* g,
                         int64_t n, float lr, float beta1, float beta2, float eps,
                         float weight_decay, int64_t step, uint16_t* p16, hipStream_t stream);

// ---- LoRA dropout -------------------------------------------------------------

// Keep mask of an [M x K] adapter input (K a multiple of 32): Philox4x32-10
// with the 64-bit seed as key and (group, offset) as counter, one 16-bit
// value per element compared with thr; bits packed [M][K/32].
hipError_t launch_dropout_mask(int64_t M, int64_t K, uint32_t thr, uint64_t seed,
                               uint64_t offset, uint32_t* mask, hipStream_t stream);

// The mask and the inverse keep probability of one linear call; a null mask
// means no dropout.
struct Dropout {
  const uint32_t* mask = nullptr;
  float keep_scale = 1.0f;
};

// ---- linear layer -----------------------------------------------------------

// Workspace carve-up for the forward and backward of one linear call.
size_t linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int r);

// Small-M forward (M <= kGemvMaxM): one launch; workgroups that form split
// partials of T = X A (a copy per XCD), and workgroups over row tiles of the
// whole K that wait for them, add s T B and write Y.
constexpr int kGemvMaxM = 16;
int64_t gemv_partial_elems(int64_t M, int64_t N, int64_t K, int r);
void set_gemv_wait_us(int64_t us);
hipError_t launch_fwd_gemv(const uint16_t* X, Nf4Weight W, const uint16_t* A,
                           const uint16_t* B, int M, int64_t N, int64_t K, int r,
                           float scale, uint16_t* Y, float* T_out, void* ws,
                           hipStream_t stream, hipEvent_t ev0 = nullptr,
                           hipEvent_t ev1 = nullptr);

// Large-M forward: T = X A, then Y = [X | s T] [W' | B^T]^T on MFMA tiles.
hipError_t launch_fwd_gemm(const uint16_t* X, Nf4Weight W, const uint16_t* A,
                           const uint16_t* B, int64_t M, int64_t N, int64_t K,
                           int r, float scale, uint16_t* Y, float* T_out, void* ws,
                           hipStream_t stream, hipEvent_t ev0 = nullptr,
                           hipEvent_t ev1 = nullptr, Dropout dr = Dropout{});

// Backward: G = dY B^T, dX = [dY | s G] [W' ; A^T], dA = s X^T G, dB = s T^T dY.
hipError_t launch_bwd(const uint16_t* dY, const uint16_t* X, const float* T,
                      Nf4Weight W, const uint16_t* A, const uint16_t* B,
                      int64_t M, int64_t N, int64_t K, int r, float scale,
                      uint16_t* dX, float* dA, float* dB, void* ws,
                      hipStream_t stream, hipEvent_t ev0 = nullptr,
                      hipEvent_t ev1 = nullptr, Dropout dr = Dropout{});

// Forward with the library's own scratch array (one per device, this many
// bytes) in place of a caller workspace.
constexpr size_t kNoAllocScratchBytes = (size_t)32 << 20;
hipError_t launch_fwd_noalloc(const uint16_t* X, Nf4Weight W, const uint16_t* A,
                              const uint16_t* B, int64_t M, int64_t N, int64_t K, int r,
                              float scale, uint16_t* Y, float* T_out, hipStream_t stream);

// Records `ev` on `stream` when it is not null (profiling hooks around the
// dominant launch of a call).
inline hipError_t record_if(hipEvent_t ev, hipStream_t stream) {
  return ev ? hipEventRecord(ev, stream) : hipSuccess;
}

}  // namespace qlora
