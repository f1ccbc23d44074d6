// Device scratch of lcd_decode_step_noalloc, for callers that cannot allocate: a
// file-scope device array (one copy per GPU, held until the process ends) and the cache
// of its device address per GPU.  Host code never passes the array's name to a kernel
// (in host code it is a stand-in, not a device address): the address is resolved here
// with hipGetSymbolAddress, once per device with that device current.
#include <hip/hip_runtime.h>

#include <mutex>

#include "lcd_internal.h"

static __device__ __align__(256) char scratch[lcd::kScratchBytes];

namespace lcd {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};
}  // namespace

hipError_t scratch_device_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255u)) return hipErrorInvalidValue;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace lcd
