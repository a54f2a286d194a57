// fp8q_api.hip -- status strings and version of the C ABI, the measurement hook, and the
// reference kernels that measurements of the path are read against.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8q.h"
#include "fp8q_launch.h"

namespace {

// Nothing: what a launch costs on this device before it does any work.
__global__ __launch_bounds__(256) void reference_empty_kernel() {}

// A plain stream with the path's 2:1 read/write mix (bf16 in, one byte per element out, as
// the group quantizer and the KV write move data): each lane reads 16 bytes with the
// non-temporal hint and writes 8, grid-stride over a grid of 4 blocks per CU.  Of the stream
// shapes measured for these byte counts (plain or non-temporal loads, 1 to 8 loads in flight
// per lane, 4 or 8 blocks per CU or one pass), this one is the fastest at the quantizer's
// 71 MB and within 2 % of the fastest at the KV write's 101 MB.  The written word depends on
// the read one, so no read is dead.
constexpr int kRefBlock = 256;
typedef unsigned ref_v4u __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(kRefBlock) void reference_stream_kernel(const ref_v4u* __restrict__ src,
                                                                     uint2* __restrict__ dst,
                                                                     int64_t n16) {
  const int64_t stride = int64_t(gridDim.x) * kRefBlock;
  for (int64_t i = int64_t(blockIdx.x) * kRefBlock + threadIdx.x; i < n16; i += stride) {
    const ref_v4u v = __builtin_nontemporal_load(src + i);
    dst[i] = make_uint2(v[0] ^ v[1], v[2] ^ v[3]);
  }
}

// The operand path of the prefill GEMM with nothing else: 512-thread workgroups, one per
// CU, copy 64 KB slices of src into LDS with the same buffer_load ... lds instructions (16
// bytes per lane, 1 KB per wave instruction), one slice landing while the next is issued and
// a barrier per slice.  Slice s reads bytes [(s * 64 KB) % span, + 64 KB), so a span that
// fits the L2 of every XCD measures the copy path from L2, a span of 1 GB from HBM.
constexpr int kLdsSlice = 65536;
typedef __attribute__((address_space(3))) void lds_void;
__global__ __launch_bounds__(512, 1) void reference_lds_stream_kernel(const uint8_t* src,
                                                                      int64_t span,
                                                                      int64_t slices) {
  __shared__ __attribute__((aligned(16))) uint8_t buf0[kLdsSlice];
  __shared__ __attribute__((aligned(16))) uint8_t buf1[kLdsSlice];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src), 0, int(span), 0x00020000);
  auto issue = [&](int64_t s, uint8_t* dst) {
    const int base = int((s * kLdsSlice) % span);
#pragma unroll
    for (int q = 0; q < 8; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + (wave + 8 * q) * 1024), 16,
                                               base + (wave + 8 * q) * 1024 + lane * 16, 0, 0,
                                               0);
  };
  int64_t s = blockIdx.x;
  if (s >= slices) return;
  issue(s, buf0);
  for (int par = 1;; par ^= 1) {
    const int64_t next = s + gridDim.x;
    if (next < slices) {
      issue(next, par ? buf1 : buf0);
      __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8): slice s landed, `next` in flight
    } else {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    }
    __syncthreads();
    if (next >= slices) break;
    s = next;
  }
}

}  // namespace

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

extern "C" int fp8q_version(void) { return 10200; }

extern "C" int fp8q_time_next_launch(hipEvent_t start, hipEvent_t stop) {
  fp8q::g_next_launch_events.start = start;
  fp8q::g_next_launch_events.stop = stop;
  return FP8Q_OK;
}

extern "C" int fp8q_reference_empty(hipStream_t stream) {
  fp8q::launch(reference_empty_kernel, dim3(1), dim3(kRefBlock), 0, stream);
  return fp8q::launch_status();
}

extern "C" int fp8q_reference_stream(const void* src, void* dst, int64_t src_bytes,
                                     hipStream_t stream) {
  if (src_bytes < 0 || src_bytes % 16 != 0) return FP8Q_EINVAL;
  if (src_bytes == 0) return FP8Q_OK;
  if (!src || !dst) return FP8Q_ENULL;
  if (!fp8q::aligned(src, 16) || !fp8q::aligned(dst, 8)) return FP8Q_EALIGN;
  fp8q::launch(reference_stream_kernel, dim3(unsigned(4 * fp8q::num_cus())), dim3(kRefBlock), 0,
               stream, static_cast<const ref_v4u*>(src), static_cast<uint2*>(dst), src_bytes / 16);
  return fp8q::launch_status();
}

extern "C" int fp8q_reference_lds_stream(const void* src, int64_t span_bytes, int64_t total_bytes,
                                         hipStream_t stream) {
  if (span_bytes < kLdsSlice || span_bytes % kLdsSlice != 0 || span_bytes > 0x7FFF0000 ||
      total_bytes < 0 || total_bytes % kLdsSlice != 0)
    return FP8Q_EINVAL;
  if (total_bytes == 0) return FP8Q_OK;
  if (!src) return FP8Q_ENULL;
  if (!fp8q::aligned(src, 16)) return FP8Q_EALIGN;
  fp8q::launch(reference_lds_stream_kernel, dim3(unsigned(fp8q::num_cus())), dim3(512), 0, stream,
               static_cast<const uint8_t*>(src), span_bytes, total_bytes / kLdsSlice);
  return fp8q::launch_status();
}
