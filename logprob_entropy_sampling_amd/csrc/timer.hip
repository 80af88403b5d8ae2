// Optional timing bracket around the main sweep kernel(s) of a scoring call:
// two HIP events recorded on the call's own stream, immediately before and
// after the sweep launches.  Host code only; process-wide state for one
// device, meant for benchmarks and profiling, not for concurrent callers.
#include <hip/hip_runtime.h>

#include "launch.h"

namespace vs {

namespace {
hipEvent_t g_ev[2] = {nullptr, nullptr};
int g_dev = -1;
bool g_on = false;
bool g_have = false;  // a start/stop pair has been recorded since the timer was enabled
}  // namespace

int timer_enable(int on) {
  if (!on) {
    g_on = false;
    return 0;
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return 1;
  if (g_ev[0] && g_dev != dev) {
    (void)hipEventDestroy(g_ev[0]);
    (void)hipEventDestroy(g_ev[1]);
    g_ev[0] = g_ev[1] = nullptr;
  }
  if (!g_ev[0]) {
    if (hipEventCreate(&g_ev[0]) != hipSuccess) return 1;
    if (hipEventCreate(&g_ev[1]) != hipSuccess) {
      (void)hipEventDestroy(g_ev[0]);
      g_ev[0] = nullptr;
      return 1;
    }
    g_dev = dev;
  }
  g_on = true;
  g_have = false;
  return 0;
}

void timer_mark(int stop, void* stream) {
  if (!g_on) return;
  if (hipEventRecord(g_ev[stop ? 1 : 0], static_cast<hipStream_t>(stream)) == hipSuccess && stop) g_have = true;
}

int timer_read_ms(float* ms) {
  if (!g_have) return 2;
  if (hipEventSynchronize(g_ev[1]) != hipSuccess) return 1;
  return hipEventElapsedTime(ms, g_ev[0], g_ev[1]) == hipSuccess ? 0 : 1;
}

}  // namespace vs
