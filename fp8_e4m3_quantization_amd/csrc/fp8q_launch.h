// fp8q_launch.h -- host-side helpers shared by the C-ABI entry points.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8q.h"

namespace fp8q {

inline bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// Grid-stride kernels never need more than this many blocks to fill 256 CUs many times.
inline int64_t clamp_grid(int64_t blocks) {
  const int64_t cap = int64_t(1) << 20;
  return blocks < 1 ? 1 : (blocks > cap ? cap : blocks);
}

// Events the next kernel launched by this host thread records when it starts and when
// it ends (set through fp8q_time_next_launch; consumed by that launch).
struct LaunchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
inline thread_local LaunchEvents g_next_launch_events;

// Every kernel of the library is enqueued through here.
template <typename Kernel, typename... Args>
inline void launch(Kernel kernel, dim3 grid, dim3 block, size_t lds, hipStream_t stream,
                   Args... args) {
  const LaunchEvents ev = g_next_launch_events;
  if (ev.start || ev.stop) {
    g_next_launch_events = LaunchEvents();
    hipExtLaunchKernelGGL(kernel, grid, block, lds, stream, ev.start, ev.stop, 0, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, args...);
  }
}

// Compute units of the current device (cached per device).
inline int num_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cus[dev]) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        v <= 0)
      v = 256;
    cus[dev] = v;
  }
  return cus[dev];
}

// Status of the launch just enqueued on this thread.
inline int launch_status() {
  return hipGetLastError() == hipSuccess ? FP8Q_OK : FP8Q_ELAUNCH;
}

}  // namespace fp8q
