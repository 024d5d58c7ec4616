/*
 * qlora.h — C ABI of the MI355X (gfx950) NF4 linear layer with a LoRA adapter.
 *
 * The library implements the frozen 4-bit linear layer of QLoRA finetuning:
 * blockwise NormalFloat-4 quantization with double quantization of the block
 * constants, the forward product with dequantization fused into a bfloat16
 * matrix product, and the backward pass that returns gradients for the input
 * and the two adapter matrices only.
 *
 * Sources (page address, title, section):
 *   ozercemkelahmet.com/tools/qlora "QLoRA", How it works, Steps 1-6, and
 *     "A worked example";
 *   crackai.dev/papers/qlora "QLoRA: Efficient Finetuning of Quantized LLMs",
 *     How It Works items 1-2 and Training Flow;
 *   ai360xpert.com/papers/qlora "QLoRA", How It Works items 1-2;
 *   fanfani.net/articles/qlora "QLoRA", "The crucial split: store in four
 *     bits, compute in sixteen".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer argument that names a tensor is a DEVICE pointer (memory of
 *   the GPU that is current on the calling thread) unless stated otherwise.
 *   The caller owns all memory; the library never allocates, frees or
 *   synchronizes, and keeps no data between calls.
 * - bfloat16 tensors are passed as uint16_t bit patterns; float tensors are
 *   IEEE binary32. All matrices are dense, row-major, contiguous.
 * - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued on
 *   it and the call returns without waiting. Calls enqueue kernel launches
 *   only (no memset, no copy, no allocation, no synchronization), so any
 *   sequence of them can be captured into a HIP graph and replayed.
 * - Return value: QLORA_OK (0) or a negative status. Arguments are validated
 *   before anything is enqueued; a failed validation has no side effects.
 *   QLORA_ERR_HIP means a launch failed; qlora_last_hip_error() then returns
 *   the hipError_t of the calling thread's last failure. Nothing prints,
 *   throws or aborts.
 * - Calls that share a workspace buffer must not overlap in time (same
 *   stream, or caller-side ordering). Otherwise calls are thread-safe: host
 *   threads may call concurrently on their own streams with their own
 *   buffers (the process state is per-device flags, set once under an
 *   atomic, recording that a kernel's LDS limit has been raised, and the
 *   scratch array of qlora_linear_fwd_noalloc with its cached address).
 *
 * The NF4 store
 * -------------
 * A tensor of `numel` values (flat, row-major) is stored in three buffers:
 *   codes     uint8 [qlora_nf4_codes_bytes(numel) = ceil(numel/2)]
 *             4-bit level indices; element 2i in the low nibble of byte i,
 *             element 2i+1 in the high nibble; an odd tail leaves the last
 *             high nibble 0.
 *   absmax_q  uint8 [qlora_nf4_num_blocks(numel) = ceil(numel/64)]
 *             8-bit code of each block's absolute maximum.
 *   absmax_s2 float [qlora_nf4_num_groups(numel) = ceil(nblocks/256)]
 *             second-level constant (maximum block constant) of each group
 *             of 256 consecutive blocks.
 * Dequantized value of element i (block b = i/64, group g = b/256):
 *   c'  = fl32( fl32(absmax_q[b] / 255) * absmax_s2[g] )
 *   w'  = fl32( NF4[code_i] * c' )
 * and the compute weight is bf16(w'), rounded to nearest even.
 *
 * The store without double quantization (ozercemkelahmet.com "QLoRA",
 * Step 2 alone: one 32-bit constant per block, 4.5 bits per weight) is
 * passed as absmax_q = NULL, and absmax_s2 then holds
 *   absmax_s2 float [qlora_nf4_num_blocks(numel)]
 *             the float32 constant (largest magnitude) of each block,
 * so that c' = absmax_s2[b]. The codes are the same in both stores. Every
 * entry point that takes a store accepts either form.
 *
 * Store types (the _ex entry points; bit flags, 0 everywhere else)
 * ----------------------------------------------------------------
 * QLORA_STORE_FP4: the levels are FP4 instead of NF4 (the 4-bit alternative
 *   that ozercemkelahmet.com "QLoRA", Common mistakes, warns not to pick
 *   without a reason; the pages do not define it): the OCP MX E2M1
 *   magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 divided by 6, sign-magnitude codes
 *   (code 8 s + m is (-1)^s E2M1(m) / 6, each level the nearest float32),
 *   so the range is [-1, 1] with an exact 0. A value takes the code of the
 *   nearest level; of two equally near, the one with an even magnitude m,
 *   then the lower code (0 goes to code 0); an all-zero block stores code 0.
 * QLORA_STORE_DQ_FP8: the 8-bit code of the block constants is the OCP E4M3
 *   code relative to a per-group scale instead of the linear code
 *   (ozercemkelahmet.com "QLoRA", Step 3 says 8 bits, not which code):
 *     S = fl32(max c / 448),  absmax_q[b] = E4M3(fl32(c / S)) (nearest,
 *     ties to even, saturating at 448; 0 when S = 0),  absmax_s2[g] = S,
 *     c' = fl32(dec(absmax_q[b]) * S).
 *   With absmax_q = NULL (no double quantization) this flag has no effect.
 * Buffers and sizes are the same for every type; w' = fl32(L[code] * c')
 * with L the type's levels in code order.
 */
#ifndef QLORA_H
#define QLORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  QLORA_OK = 0,
  QLORA_ERR_INVALID_ARG = -1, /* null required pointer, bad size, numel mismatch */
  QLORA_ERR_UNSUPPORTED = -2, /* K or N not a multiple of 64, r outside [1, 256],
                                 a dimension above 2^30, misaligned pointer */
  QLORA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  QLORA_ERR_HIP = -4          /* a HIP launch failed; see qlora_last_hip_error() */
};

#define QLORA_STORE_NF4 0
#define QLORA_STORE_FP4 1
#define QLORA_STORE_DQ_FP8 2

#define QLORA_NF4_BLOCK 64
#define QLORA_NF4_GROUP 256
#define QLORA_MAX_RANK 256
/* Largest adapter rank of qlora_linear_bwd_dropout with an input gradient. */
#define QLORA_MAX_DROPOUT_RANK 192

/* ---- sizes of the NF4 store (host functions, no GPU work) ---------------- */

/* ceil(numel / 2); -1 if numel < 0. */
int64_t qlora_nf4_codes_bytes(int64_t numel);
/* ceil(numel / 64); -1 if numel < 0. */
int64_t qlora_nf4_num_blocks(int64_t numel);
/* ceil(ceil(numel / 64) / 256); -1 if numel < 0. */
int64_t qlora_nf4_num_groups(int64_t numel);

/* The 16 NF4 levels as used by the kernels, ascending (host copy).
 * They are the float32 roundings of standard-normal quantiles at equal
 * probability steps within each half, scaled so the endpoints are -1 and +1
 * with an exact 0 (crackai.dev "QLoRA: Efficient Finetuning of Quantized
 * LLMs", How It Works item 1; ozercemkelahmet.com "QLoRA", Why NormalFloat).
 * `levels` is a HOST pointer to 16 floats. */
void qlora_nf4_codebook(float* levels);

/* ---- quantization ---------------------------------------------------------
 * qlora_nf4_quantize — blockwise NF4 quantization with double quantization
 * (ozercemkelahmet.com "QLoRA", How it works, Steps 1-3 and "A worked
 * example"; ai360xpert.com "QLoRA", How It Works item 2).
 *
 *   w          device, bf16 [numel]            input weights (flat row-major)
 *   numel      > 0
 *   codes      device, uint8 [ceil(numel/2)]    output, see "The NF4 store"
 *   absmax_q   device, uint8 [ceil(numel/64)]   output
 *   absmax_s2  device, float [num_groups]       output
 * Per block of 64: c = max|w|; each value maps to the index of the nearest
 * level of fl32(w / c) (ties to the lower index; c = 0 gives index 7, the
 * level 0). Per group of 256 constants: s2 = max c and
 * absmax_q = round_half_even(255 * fl32(c / s2)) (0 when s2 = 0).
 * A short final block or group takes its maximum over the values present.
 * absmax_q = NULL writes the store without double quantization instead:
 * absmax_s2 [ceil(numel/64)] receives each block's c (same codes).
 * Errors: INVALID_ARG for a null w, codes or absmax_s2, or numel <= 0;
 * UNSUPPORTED if `w` is not 2-byte aligned or `codes` / `absmax_s2` not
 * 4-byte aligned. Needs no workspace. */
int qlora_nf4_quantize(const uint16_t* w, int64_t numel, uint8_t* codes,
                       uint8_t* absmax_q, float* absmax_s2, void* stream);

/* qlora_nf4_quantize_ex — qlora_nf4_quantize for any store type (see
 * "Store types"); store_type 0 is qlora_nf4_quantize.
 * Errors: as qlora_nf4_quantize; INVALID_ARG for a store_type outside
 * [0, 3]. */
int qlora_nf4_quantize_ex(const uint16_t* w, int64_t numel, uint8_t* codes,
                          uint8_t* absmax_q, float* absmax_s2, int32_t store_type,
                          void* stream);

/* qlora_nf4_dequantize — expand a store to float32 w' (the formula in
 * "The NF4 store"; ozercemkelahmet.com "QLoRA", "A worked example" step 4).
 *   out        device, float [numel]
 * Errors: INVALID_ARG for a null pointer or numel <= 0; UNSUPPORTED if
 * `codes` or `absmax_s2` is not 4-byte aligned or `out` not 16-byte
 * aligned. */
int qlora_nf4_dequantize(const uint8_t* codes, const uint8_t* absmax_q,
                         const float* absmax_s2, int64_t numel, float* out,
                         void* stream);

/* qlora_nf4_dequantize_bf16 — as above, but writes the bf16 compute weight
 * bf16(w') (ozercemkelahmet.com "QLoRA", Step 5: the block is dequantized
 * into the compute type). `out` is device uint16 [numel], 16-byte aligned. */
int qlora_nf4_dequantize_bf16(const uint8_t* codes, const uint8_t* absmax_q,
                              const float* absmax_s2, int64_t numel,
                              uint16_t* out, void* stream);

/* The two dequantizations for any store type (store_type before the
 * output); errors as above, INVALID_ARG for a store_type outside [0, 3]. */
int qlora_nf4_dequantize_ex(const uint8_t* codes, const uint8_t* absmax_q,
                            const float* absmax_s2, int64_t numel, int32_t store_type,
                            float* out, void* stream);
int qlora_nf4_dequantize_bf16_ex(const uint8_t* codes, const uint8_t* absmax_q,
                                 const float* absmax_s2, int64_t numel, int32_t store_type,
                                 uint16_t* out, void* stream);

/* qlora_nf4_merge — the adapter folded into a 16-bit copy of the frozen
 * weight (ozercemkelahmet.com "QLoRA", How it works, Step 8: save and use:
 * dequantize the base to 16 bits and merge the adapter; same page, "Merging
 * after QLoRA"). With A [K x r] and B [r x N] as in the linear calls, a
 * forward pass computes X (W' + s (A B)^T)^T, so
 *   out[n][k] = bf16( w'[n][k] + scale * sum_j A[k][j] B[j][n] )
 * in this order: the sum in float32 from j = 0 upward (each product of two
 * bf16 values is exact), then fl32(scale * sum), fl32(w' + that), one
 * round-to-nearest-even to bf16. Deterministic.
 *   codes, absmax_q, absmax_s2   the store of W [N x K] (numel = N*K)
 *   A        device bf16 [K x r];  B  device bf16 [r x N]   (2-byte aligned)
 *   out      device bf16 [N x K], 16-byte aligned, written
 * Errors: INVALID_ARG for a null pointer or N, K <= 0; UNSUPPORTED if K is
 * not a multiple of 64, r is outside [1, 256], N or K exceeds 2^30 (or N
 * needs more than 65535 row tiles of 64), `codes` is not 16-byte aligned,
 * `absmax_s2` not 4-byte aligned or `out` not 16-byte aligned. */
int qlora_nf4_merge(const uint8_t* codes, const uint8_t* absmax_q, const float* absmax_s2,
                    int64_t N, int64_t K, const uint16_t* A, const uint16_t* B, int32_t r,
                    float scale, uint16_t* out, void* stream);
/* ... for any store type (INVALID_ARG for a store_type outside [0, 3]). */
int qlora_nf4_merge_ex(const uint8_t* codes, const uint8_t* absmax_q, const float* absmax_s2,
                       int64_t N, int64_t K, const uint16_t* A, const uint16_t* B, int32_t r,
                       float scale, int32_t store_type, uint16_t* out, void* stream);

/* qlora_adamw_step — one AdamW step for adapter parameters, in place
 * (ozercemkelahmet.com "QLoRA", "Practical guidance and best practices",
 * Optimizer and schedule: AdamW with paged state in 8 or 32 bits; same
 * page, "How it works", Step 7). Float32 parameters p, moments m and v, gradient g (for
 * example dA or dB of qlora_linear_bwd), n elements each; step t >= 1 counts
 * from 1. Each operation is one float32 operation rounded on its own, in
 * this order (host constants computed in float64 and rounded once):
 *   lw = lr*wd, c1 = 1 - beta1^t, c2 = 1 - beta2^t
 *   p1 = p - lw*p
 *   m  = beta1*m + (1-beta1)*g
 *   v  = beta2*v + (1-beta2)*(g*g)
 *   p  = p1 - lr*((m/c1) / (sqrt(v/c2) + eps))
 * p_bf16 (optional, device uint16 [n]) receives bf16(p), the copy that the
 * linear calls take as A or B.
 * Host-resident state (the paged optimizer of ozercemkelahmet.com "QLoRA",
 * How it works, Step 7, keeps optimizer state in host memory when the
 * device runs short): m and v may be pinned host memory from hipHostMalloc,
 * mapped into the device's address space, passed as the address that
 * hipHostGetDevicePointer returns. The kernel then reads and writes the
 * moments in place over the host link (no copy, no managed memory, no
 * demand paging); results are the same bit for bit. p, g and p_bf16 stay
 * device memory.
 * Errors: INVALID_ARG for a null pointer, n <= 0, step < 1, beta outside
 * [0, 1) or eps <= 0; UNSUPPORTED for float arrays not 4-byte aligned or
 * p_bf16 not 2-byte aligned. */
int qlora_adamw_step(float* p, float* m, float* v, const float* g, int64_t n, float lr,
                     float beta1, float beta2, float eps, float weight_decay, int64_t step,
                     uint16_t* p_bf16, void* stream);

/* qlora_adamw8_step — qlora_adamw_step with 8-bit moments (the pages'
 * recipe trains with a paged 8-bit AdamW: ozercemkelahmet.com "QLoRA",
 * "A code example with common libraries", Training arguments, and "Practical
 * guidance and best practices", Optimizer and schedule; the pages do not say how the state is
 * held in 8 bits). Each moment is kept per block of 256 parameters (block
 * b = i / 256, the last one short) as 8-bit floating-point codes of the OCP
 * 8-bit float formats and one float32 scale:
 *   m8       device uint8 [n]            E4M3 codes of m (bias 7, max 448)
 *   m_scale  device float [ceil(n/256)]  scale of m per block
 *   v8       device uint8 [n]            E5M2 codes of v (bias 15, max 57344)
 *   v_scale  device float [ceil(n/256)]  scale of v per block
 * all zero before the first step. One step, every operation one float32
 * operation rounded on its own:
 *   m = dec(m8) * m_scale[b],  v = dec(v8) * v_scale[b]
 *   the float32 AdamW step of qlora_adamw_step on (p, m, v, g)
 *   m_scale[b] = max_block |m| / 448,   v_scale[b] = max_block v / 57344
 *   m8 = enc(m / m_scale[b]),  v8 = enc(v / v_scale[b])  (0 when the scale is 0)
 * enc rounds to the nearest code, ties to the even code, saturating at the
 * largest finite one. 18 bytes of traffic per parameter against 30 for the
 * float32 state (with the bf16 copy).
 * m8, m_scale, v8 and v_scale may be pinned host memory as m and v of
 * qlora_adamw_step.
 * Errors: as qlora_adamw_step (m8 and v8 need no alignment; the scales are
 * float arrays). */
int qlora_adamw8_step(float* p, uint8_t* m8, float* m_scale, uint8_t* v8, float* v_scale,
                      const float* g, int64_t n, float lr, float beta1, float beta2, float eps,
                      float weight_decay, int64_t step, uint16_t* p_bf16, void* stream);

/* ---- the linear layer ------------------------------------------------------
 * Shapes: X [M x K], frozen weight W [N x K] in the NF4 store (numel = N*K,
 * blocks run along K), A [K x r], B [r x N], Y and dY [M x N].
 * scale = alpha / r is computed by the caller.
 *
 * Workspace: `ws` is device memory of at least
 *   qlora_linear_workspace_bytes(M, N, K, r)
 * bytes, 256-byte aligned, owned by the caller; it may be reused between
 * calls that do not overlap. Its contents on entry do not matter. The query
 * returns 0 for a shape or rank that the linear calls reject. */
size_t qlora_linear_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t r);

/* qlora_linear_fwd — Y = X bf16(W')^T + scale * (X A) B
 * (ozercemkelahmet.com "QLoRA", Step 5, written there in column form
 * y = dequant(W) x + (alpha/r) B(Ax); crackai.dev "QLoRA: Efficient
 * Finetuning of Quantized LLMs", Training Flow: dequantize to bf16 on the fly
 * and compute with LoRA).
 *   X        device bf16 [M x K]
 *   codes, absmax_q, absmax_s2   the NF4 store of W, numel = N*K
 *   A        device bf16 [K x r];  B  device bf16 [r x N]
 *   Y        device bf16 [M x N]   output (bf16 of the float32 accumulation)
 *   T_out    device float [M x r]  optional output: T = X A (for the
 *                                  backward); NULL to skip
 * Products of bf16 values accumulate in float32. M <= 16 takes a
 * memory-bound GEMV path (one launch: workgroups that form split partials
 * of X A, and one workgroup per 16 weight rows over the whole K that waits
 * for them, adds the adapter term and writes Y; see qlora_gemv_wait_limit);
 * larger M takes an MFMA GEMM path. Calls capture into a HIP graph (no
 * memset, no allocation).
 * Errors: INVALID_ARG (null X/codes/absmax/A/B/Y, non-positive M, N, K);
 * UNSUPPORTED (K or N not a multiple of 64, r outside [1, 256], M above
 * 2^30, N or K above 2^21, M N or M K at or above 2^30, N K at or above
 * 2^32 (the kernels address operands with 32-bit offsets); codes, X or B
 * not 16-byte aligned, A or Y not 2-byte aligned, absmax_s2 or T_out not
 * 4-byte aligned, ws not 256-byte aligned);
 * WORKSPACE (ws NULL or ws_bytes below the query). */
int qlora_linear_fwd(const uint16_t* X, const uint8_t* codes,
                     const uint8_t* absmax_q, const float* absmax_s2,
                     const uint16_t* A, const uint16_t* B, int64_t M,
                     int64_t N, int64_t K, int32_t r, float scale,
                     uint16_t* Y, float* T_out, void* ws, size_t ws_bytes,
                     void* stream);

/* qlora_linear_fwd_ex — qlora_linear_fwd on a store of any type (the GEMV
 * and the MFMA path take the type's levels and constant code); errors as
 * qlora_linear_fwd, INVALID_ARG for a store_type outside [0, 3]. */
int qlora_linear_fwd_ex(const uint16_t* X, const uint8_t* codes,
                        const uint8_t* absmax_q, const float* absmax_s2,
                        const uint16_t* A, const uint16_t* B, int64_t M,
                        int64_t N, int64_t K, int32_t r, float scale,
                        uint16_t* Y, float* T_out, void* ws, size_t ws_bytes,
                        int32_t store_type, void* stream);

/* qlora_linear_bwd — gradients through the dequantized frozen weight into
 * the input and the adapter; no gradient for the 4-bit weight
 * (ozercemkelahmet.com "QLoRA", Step 6; crackai.dev "QLoRA: Efficient
 * Finetuning of Quantized LLMs", Training Flow; ai360xpert.com "QLoRA",
 * The Idea):
 *   G  = dY B^T                   [M x r]
 *   dX = dY bf16(W') + scale G A^T
 *   dA = scale X^T G              [K x r]
 *   dB = scale T^T dY             [r x N],  T = X A
 *   dY       device bf16 [M x N]
 *   X        device bf16 [M x K]
 *   T        device float [M x r] from qlora_linear_fwd, or NULL to recompute
 *   dX       device bf16 [M x K] output, or NULL to skip the input gradient
 *   dA       device float [K x r] output (overwritten, not accumulated)
 *   dB       device float [r x N] output (overwritten, not accumulated)
 * Errors: as qlora_linear_fwd, with dY 16-byte aligned, dX 2-byte and
 * T, dA, dB 4-byte aligned; dA and dB must not be NULL. */
int qlora_linear_bwd(const uint16_t* dY, const uint16_t* X, const float* T,
                     const uint8_t* codes, const uint8_t* absmax_q,
                     const float* absmax_s2, const uint16_t* A,
                     const uint16_t* B, int64_t M, int64_t N, int64_t K,
                     int32_t r, float scale, uint16_t* dX, float* dA,
                     float* dB, void* ws, size_t ws_bytes, void* stream);

/* qlora_linear_fwd_noalloc — qlora_linear_fwd without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation). The
 * scratch memory is a fixed device array of QLORA_NOALLOC_SCRATCH_BYTES that
 * the library holds on each GPU it runs on until the process ends; the call
 * itself allocates and frees nothing. Same kernels, same results bit for bit
 * as qlora_linear_fwd. Every call on one GPU shares that GPU's array: calls
 * that overlap in time on one GPU (concurrent streams or host threads) race
 * and give undefined results; calls ordered on one stream are safe. The
 * array's contents on entry do not matter.
 * Errors: as qlora_linear_fwd; WORKSPACE when the shape needs more than
 * QLORA_NOALLOC_SCRATCH_BYTES (qlora_linear_workspace_bytes above it, e.g.
 * beyond the 8192-token, 22016-wide linear at r = 64); QLORA_ERR_HIP also
 * when the array's device address cannot be obtained on the current GPU. */
#define QLORA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int qlora_linear_fwd_noalloc(const uint16_t* X, const uint8_t* codes,
                             const uint8_t* absmax_q, const float* absmax_s2,
                             const uint16_t* A, const uint16_t* B, int64_t M,
                             int64_t N, int64_t K, int32_t r, float scale,
                             uint16_t* Y, float* T_out, void* stream);

/* qlora_linear_bwd_ex — qlora_linear_bwd on a store of any type; errors as
 * qlora_linear_bwd, INVALID_ARG for a store_type outside [0, 3]. */
int qlora_linear_bwd_ex(const uint16_t* dY, const uint16_t* X, const float* T,
                        const uint8_t* codes, const uint8_t* absmax_q,
                        const float* absmax_s2, const uint16_t* A,
                        const uint16_t* B, int64_t M, int64_t N, int64_t K,
                        int32_t r, float scale, uint16_t* dX, float* dA,
                        float* dB, void* ws, size_t ws_bytes, int32_t store_type,
                        void* stream);

/* ---- profiling variants ------------------------------------------------------
 * Identical to qlora_linear_fwd / qlora_linear_bwd, and in addition record
 * the caller's hipEvent_t `ev_begin` and `ev_end` (created by the caller,
 * either may be NULL) on `stream` immediately before and after the launch of
 * the call's dominant kernel: the fused NF4 product kernel of the forward
 * (the GEMV for M <= 16, the MFMA contraction otherwise) and the fused
 * input-gradient contraction of the backward (no events when dX is NULL).
 * For measuring that kernel's duration with hipEventElapsedTime. */
int qlora_linear_fwd_profiled(const uint16_t* X, const uint8_t* codes,
                              const uint8_t* absmax_q, const float* absmax_s2,
                              const uint16_t* A, const uint16_t* B, int64_t M,
                              int64_t N, int64_t K, int32_t r, float scale,
                              uint16_t* Y, float* T_out, void* ws,
                              size_t ws_bytes, void* stream, void* ev_begin,
                              void* ev_end);
int qlora_linear_bwd_profiled(const uint16_t* dY, const uint16_t* X,
                              const float* T, const uint8_t* codes,
                              const uint8_t* absmax_q, const float* absmax_s2,
                              const uint16_t* A, const uint16_t* B, int64_t M,
                              int64_t N, int64_t K, int32_t r, float scale,
                              uint16_t* dX, float* dA, float* dB, void* ws,
                              size_t ws_bytes, void* stream, void* ev_begin,
                              void* ev_end);

/* ---- LoRA dropout -------------------------------------------------------------
 * Dropout on the input of the adapter path only (ozercemkelahmet.com
 * "QLoRA": the LoraConfig of "A code example with common libraries" trains
 * with lora_dropout = 0.05; "Practical guidance and best practices", Adapter
 * settings: a small dropout rate when data is scarce). With a keep mask over
 * X and f the inverse keep probability,
 *   D(X) = (X o keep) f,   Y = X bf16(W')^T + scale * (D(X) A) B,
 * the frozen-weight product sees X unchanged (inverted dropout).
 *
 * Keep mask: uint32 [M][K/32], bit j of word w of row m is element
 * (m, 32 w + j); 1 = kept. qlora_dropout_mask draws it; a caller that needs
 * the mask again (the backward, or a recomputed forward under gradient
 * checkpointing) may keep it (M K / 8 bytes) or draw it again from the same
 * seed and offset.
 *
 * Drop probability realized: thr / 2^16 with thr = floor(p 2^16 + 1/2)
 * (0.0500030518 for p = 0.05); f = 2^16 / (2^16 - thr), rounded to float. */

/* qlora_dropout_mask — keep mask of an [M x K] adapter input.
 * Random numbers: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
 * random numbers: as easy as 1, 2, 3", SC'11) with key = seed (low word
 * first) and counter = (g mod 2^32, g div 2^32, offset mod 2^32,
 * offset div 2^32) for group g of eight consecutive elements of X in
 * row-major order; output word w gives the 16-bit values of elements
 * 8g + 2w (low half) and 8g + 2w + 1 (high half); an element is kept when
 * its value is at least thr. The mask of a given (seed, offset, p) depends
 * only on each element's flat index m K + k.
 *   mask   device uint32 [M x K/32] output
 * Errors: INVALID_ARG (null mask, M or K not positive, p outside [0, 1) or
 * NaN); UNSUPPORTED (K not a multiple of 32, p rounding to thr = 2^16,
 * M K above 2^40, mask not 4-byte aligned). */
int qlora_dropout_mask(int64_t M, int64_t K, float p, uint64_t seed, uint64_t offset,
                       uint32_t* mask, void* stream);

/* qlora_linear_fwd_dropout — qlora_linear_fwd with LoRA dropout:
 *   Y = X bf16(W')^T + scale * T B,   T = D(X) A
 *   keep_mask  device uint32 [M x K/32] from qlora_dropout_mask (p the same)
 *   T_out      optional: T = D(X) A, which qlora_linear_bwd_dropout takes
 * Every M takes the MFMA path (the mask enters the X A contraction).
 * Errors: as qlora_linear_fwd; INVALID_ARG also for a null keep_mask or p
 * outside [0, 1); UNSUPPORTED for p rounding to certain dropping or a
 * keep_mask not 4-byte aligned. */
int qlora_linear_fwd_dropout(const uint16_t* X, const uint8_t* codes,
                             const uint8_t* absmax_q, const float* absmax_s2,
                             const uint16_t* A, const uint16_t* B, int64_t M,
                             int64_t N, int64_t K, int32_t r, float scale,
                             const uint32_t* keep_mask, float p, uint16_t* Y,
                             float* T_out, void* ws, size_t ws_bytes, void* stream);

/* qlora_linear_bwd_dropout — qlora_linear_bwd with LoRA dropout (the chain
 * rule through D):
 *   G  = dY B^T
 *   dX = dY bf16(W') + scale * ((G A^T) o keep) f
 *   dA = scale * D(X)^T G,   dB = scale * T^T dY,   T = D(X) A
 *   T  the forward's T_out, or NULL to recompute it from X and the mask
 * Errors: as qlora_linear_bwd and qlora_linear_fwd_dropout; UNSUPPORTED
 * also for r above QLORA_MAX_DROPOUT_RANK when dX is requested (the masked
 * adapter columns of dX are summed from LDS stages that hold at most three
 * 64-wide rank steps). */
int qlora_linear_bwd_dropout(const uint16_t* dY, const uint16_t* X, const float* T,
                             const uint8_t* codes, const uint8_t* absmax_q,
                             const float* absmax_s2, const uint16_t* A,
                             const uint16_t* B, int64_t M, int64_t N, int64_t K,
                             int32_t r, float scale, const uint32_t* keep_mask, float p,
                             uint16_t* dX, float* dA, float* dB, void* ws,
                             size_t ws_bytes, void* stream);

/* qlora_gemv_wait_limit — how long, in microseconds, the row-tile
 * workgroups of a small-M forward (M <= 16) wait for the workgroups of the
 * same launch that form T = X A, before forming T themselves; the default,
 * 200, is far beyond the few microseconds those take. 0: no T workgroups
 * are launched and every row-tile workgroup forms T itself (slower, the
 * same results bit for bit). Host state shared by all threads; applies to
 * calls issued after it returns. Errors: INVALID_ARG for a value below 0 or
 * above 1000000. */
int qlora_gemv_wait_limit(int64_t microseconds);

/* ---- diagnostics ------------------------------------------------------------ */

/* Static text for a status code. */
const char* qlora_status_string(int status);
/* hipError_t of the calling thread's last QLORA_ERR_HIP (0 if none). */
int qlora_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_H */
