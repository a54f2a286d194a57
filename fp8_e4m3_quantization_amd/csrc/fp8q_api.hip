// fp8q_api.hip -- status strings and version of the C ABI.
#include "fp8q.h"
#include "fp8q_launch.h"

extern "C" const char* fp8q_strerror(int status) {
  switch (status) {
    case FP8Q_OK: return "ok";
    case FP8Q_EINVAL: return "invalid argument: a size, stride or scale is outside the contract";
    case FP8Q_ENULL: return "a required pointer is NULL";
    case FP8Q_EALIGN: return "a pointer or stride breaks the documented alignment";
    case FP8Q_ELAUNCH: return "the HIP runtime rejected the kernel launch";
    case FP8Q_EHIP: return "a HIP runtime call (allocation, copy or synchronization) failed";
    case FP8Q_ESTATE: return "calibrator used against its contract (e.g. from another device)";
    default: return "unknown status";
  }
}

extern "C" int fp8q_version(void) { return 10000; }

extern "C" int fp8q_time_next_launch(hipEvent_t start, hipEvent_t stop) {
  fp8q::g_next_launch_events.start = start;
  fp8q::g_next_launch_events.stop = stop;
  return FP8Q_OK;
}
