// Sampling-transform support (placeholder until the kernel lands).
#include "common.h"
#include "launch.h"

namespace vs {

int launch_transforms(const uint16_t*, int64_t, int64_t, int64_t, const float*, float, const int32_t*, const float*,
                      const float*, const int64_t*, float*, float*, uint8_t*, int32_t*, float*, int32_t*, int64_t*,
                      int64_t, float*, void*) {
  return -1;
}

}  // namespace vs
