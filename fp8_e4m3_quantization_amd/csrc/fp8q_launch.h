// fp8q_launch.h -- host-side helpers shared by the C-ABI entry points.
#pragma once
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

// Status of the launch just enqueued on this thread.
inline int launch_status() {
  return hipGetLastError() == hipSuccess ? FP8Q_OK : FP8Q_ELAUNCH;
}

}  // namespace fp8q
