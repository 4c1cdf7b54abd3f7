// Per-device runtime state of the library: the compute-unit count the planners size
// their grids for, read once per device (std::call_once) with that device current and
// never changed afterwards, so calls stay thread-safe.
#include <hip/hip_runtime.h>

#include <mutex>

#include "sa_launch.h"

namespace sa {

namespace {

constexpr int kMaxDevices = 64;

int current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
  return dev;
}

std::once_flag g_cu_once[kMaxDevices];
int g_cus[kMaxDevices];

}  // namespace

int device_cu_count() {
  const int dev = current_device();
  if (dev < 0) return 0;
  std::call_once(g_cu_once[dev], [dev]() {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) v = 0;
    g_cus[dev] = v > 0 ? v : 0;
  });
  return g_cus[dev];
}

}  // namespace sa
