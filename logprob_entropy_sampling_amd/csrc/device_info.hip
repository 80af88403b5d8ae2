// Per-device facts the launchers size their grids by (host code only).
#include <hip/hip_runtime.h>

#include <atomic>

#include "launch.h"

namespace vs {

int device_cu_count(int* ncu) {
  // Cached per device.  Every writer stores the same value, and the atomic
  // makes the concurrent first calls on several threads well defined.
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return int(hipErrorInvalidDevice);
  int n = dev < 64 ? cache[dev].load(std::memory_order_relaxed) : 0;
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return int(hipErrorInvalidDevice);
    if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  }
  *ncu = n;
  return 0;
}

}  // namespace vs
