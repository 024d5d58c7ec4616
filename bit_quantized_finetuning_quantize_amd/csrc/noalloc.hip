// The forward without a caller workspace: its scratch memory is a fixed
// array in device memory that the library holds (one per GPU it runs on,
// until the process ends), for callers that cannot allocate.
//
// The array's name is a host-side stand-in in host code: its device address
// is looked up once per device with hipGetSymbolAddress (with that device
// current) and that address is what the kernels receive, exactly as they
// receive a caller's workspace in qlora_linear_fwd.
#include "kernels.h"

#include <atomic>
#include <mutex>

namespace qlora {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of this device's scratch array; null on failure (*err set).
void* scratch_of_current_device(hipError_t* err) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) { *err = e; return nullptr; }
  if (dev < 0 || dev >= kMaxDevices) { *err = hipErrorInvalidDevice; return nullptr; }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) { *err = e != hipSuccess ? e : hipErrorInvalidSymbol; return nullptr; }
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

hipError_t launch_fwd_noalloc(const uint16_t* X, Nf4Weight W, const uint16_t* A,
                              const uint16_t* B, int64_t M, int64_t N, int64_t K, int r,
                              float scale, uint16_t* Y, float* T_out, hipStream_t stream) {
  hipError_t e = hipSuccess;
  void* ws = scratch_of_current_device(&e);
  if (!ws) return e;
  if (M <= kGemvMaxM)
    return launch_fwd_gemv(X, W, A, B, (int)M, N, K, r, scale, Y, T_out, ws, stream);
  return launch_fwd_gemm(X, W, A, B, M, N, K, r, scale, Y, T_out, ws, stream);
}

}  // namespace qlora
