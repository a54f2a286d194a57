// fp8q_launch.h -- host-side helpers shared by the C-ABI entry points.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>

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

// Status of the last launch this host thread enqueued through launch().
inline thread_local hipError_t g_last_launch = hipSuccess;

// Every kernel of the library is enqueued through here.  The arguments are converted to the
// kernel's own parameter types and handed to hipLaunchKernel / hipExtLaunchKernel, whose
// return value is this launch's status (an error left by an earlier, unrelated HIP call on
// the thread is neither reported nor cleared).
template <typename... KArgs, typename... Args>
inline void launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds,
                   hipStream_t stream, Args... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count");
  std::tuple<KArgs...> packed(static_cast<KArgs>(args)...);
  void* argv[sizeof...(KArgs) + 1];
  std::apply([&](auto&... a) {
    int i = 0;
    ((argv[i++] = static_cast<void*>(&a)), ...);
  }, packed);
  const LaunchEvents ev = g_next_launch_events;
  if (ev.start || ev.stop) {
    g_next_launch_events = LaunchEvents();
    g_last_launch = hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv,
                                       lds, stream, ev.start, ev.stop, 0);
  } else {
    g_last_launch =
        hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, lds, stream);
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
inline int launch_status() { return g_last_launch == hipSuccess ? FP8Q_OK : FP8Q_ELAUNCH; }

}  // namespace fp8q
