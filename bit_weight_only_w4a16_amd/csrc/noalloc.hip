// awq_gemm_noalloc: awq_gemm for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// awq_gemm's workspace (K split partial sums at small M, the once-per-call X' of the
// prefill kernel) lives here in a file-scope device array instead of a caller buffer.
// Each GPU the library runs on holds its own copy of the array until the process ends.
// In host code the array's name only stands in for the symbol: its device address is
// looked up once per device with hipGetSymbolAddress and only that address is passed to
// kernels. No call here allocates or frees memory.
#include "../../include/awq.h"
#include "awq_internal.hpp"

#include <atomic>
#include <mutex>

namespace {

constexpr size_t kScratchBytes = size_t{64} << 20;  // 64 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_setup;

// The device address of `scratch` on the current device (looked up on the first call on
// that device, with that device current); NULL if the lookup fails.
void* scratch_on_current_device(int* status) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *status = AWQ_ERR_HIP;
    return nullptr;
  }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_setup);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      *status = AWQ_ERR_HIP;
      return nullptr;
    }
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" {

int awq_gemm_noalloc(const uint16_t* x, const uint16_t* inv_s_c, const void* packed, int64_t M,
                     int64_t N, int64_t K, int32_t group, int32_t fmt, uint16_t* y,
                     hipStream_t stream) {
  // the checks of awq_gemm (the scratch stands in for the workspace, checked below)
  const int rc = awq::check_product(x, inv_s_c, packed, M, N, K, group, fmt, y, nullptr, 0);
  if (rc != AWQ_OK) return rc;
  if (M == 0) return AWQ_OK;
  const size_t need = awq_workspace_bytes(M, N, K, group);
  if (need > kScratchBytes) return AWQ_ERR_WORKSPACE;
  int status = AWQ_OK;
  void* ws = need > 0 ? scratch_on_current_device(&status) : nullptr;
  if (status != AWQ_OK) return status;
  return awq_gemm(x, inv_s_c, packed, M, N, K, group, fmt, y, ws, ws != nullptr ? kScratchBytes : 0,
                  stream);
}

}  // extern "C"
