// lce_noalloc.hip - lce_backward without a caller-supplied workspace, for
// callers that cannot allocate device memory (code under stream capture,
// serving loops, harnesses that forbid allocation).
//
// The workspace lives in a file-scope device array, `scratch`, of
// kStaticScratchBytes.  Each GPU the library runs on holds its own copy until
// the process ends.  In host code `scratch` names a host-side stand-in, not
// device memory, so the device address of each GPU's copy is looked up once
// per device with hipGetSymbolAddress and only that address is ever handed
// to a kernel.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "lce.h"

namespace {

constexpr size_t kStaticScratchBytes = LCE_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) char scratch[kStaticScratchBytes];

std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current device's copy of `scratch`, or nullptr if it
// cannot be had (no device, or the symbol lookup failed).
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return nullptr;
    p = addr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" lce_status_t lce_backward_static(const lce_problem_t* p, const void* hidden,
                                            const void* weight, const int32_t* targets,
                                            const float* lse, const float* grad_out,
                                            float* d_hidden, float* d_weight,
                                            hipStream_t stream) {
  const size_t need = lce_workspace_bytes(p);
  if (need == 0) return LCE_ERR_INVALID_VALUE;
  if (need > kStaticScratchBytes) return LCE_ERR_WORKSPACE;
  void* ws = scratch_ptr();
  if (!ws) return LCE_ERR_LAUNCH;
  // The backward writes every workspace byte it later reads (the control
  // block, then each gradient strip before its GEMMs), so the array needs no
  // clearing between calls.
  return lce_backward(p, hidden, weight, targets, lse, grad_out, d_hidden, d_weight, ws,
                      kStaticScratchBytes, stream);
}
