// static_scratch.hip -- the workspace of mr_route_align_noalloc, the route +
// align entry point that allocates nothing: a file-scope device array of
// kScratchBytes, one copy per GPU, held until the process ends.
//
// In host code `scratch` names a host-side stand-in, not the device array:
// its device address comes from hipGetSymbolAddress, looked up once per
// device (with that device current) and kept per device.  Only that address
// is ever handed to a kernel or a fill.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "kernels.h"

namespace {

static __device__ __align__(256) uint8_t scratch[mr::kScratchBytes];

std::atomic<void *> g_scratch_ptr[mr::kMaxDevices];  // device address per device, null until looked up
std::mutex g_scratch_mu;

}  // namespace

namespace mr {

hipError_t scratch_setup(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (g_scratch_ptr[dev].load(std::memory_order_acquire)) return hipSuccess;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev].load(std::memory_order_relaxed)) return hipSuccess;
  void *ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (!ptr || (reinterpret_cast<uintptr_t>(ptr) & 255u) != 0) return hipErrorInvalidSymbol;
  g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  return hipSuccess;
}

void *scratch_ptr(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  return g_scratch_ptr[dev].load(std::memory_order_acquire);
}

}  // namespace mr
