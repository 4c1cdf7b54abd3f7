// Scratch of the no-allocation decode entry point (sink_attn_decode_noalloc): a
// file-scope device array that stands in for the caller's workspace, for callers that
// cannot allocate (code under graph capture, tight serving loops).  Each GPU holds its
// own copy for the life of the process.  In host code the array's name is only a
// handle, not a device address: the address is looked up once per device, with that
// device current, and only that address is ever passed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "sa_launch.h"

static __device__ __align__(256) unsigned char scratch[sa::kNoAllocScratchBytes];

namespace sa {

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev]() {
    void* p = nullptr;
    const hipError_t r = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_err[dev] = r;
    g_ptr[dev] = (r == hipSuccess) ? p : nullptr;
  });
  *ptr = g_ptr[dev];
  return g_err[dev];
}

}  // namespace sa
