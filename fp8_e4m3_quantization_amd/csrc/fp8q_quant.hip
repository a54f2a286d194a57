// fp8q_quant.hip -- per-token 1x128 group quantization (bf16 -> E4M3 + fp32 scales),
// the 128x128 weight block quantizer and the element-wise binary32 -> E4M3 encoder.
//
// Group quant (fp8_act_quant.rs page, module doc: one scale per 128-wide K-group of a
// token row; every variant must produce the same bytes).  The pages' two CUDA kernels
// spend a 128-thread CTA, or 16 threads, on each group.  Here a [m, k] bf16 matrix with
// k % 128 == 0 is a flat run of m*k/128 groups of 256 contiguous bytes, and one gfx950
// wave64 quantizes 8 consecutive groups: 8 lanes per group, 16 bf16 (32 bytes) per lane.
//   - loads: two 16-byte loads per lane, the wave reads 2 KB contiguous;
//   - amax: max of 16 magnitudes per lane, then 3 DPP steps inside the 8-lane group
//     (no LDS, no barrier);
//   - scale s = max(amax, 1e-10)/448 and y = RN(1/s) once per group (all 8 lanes);
//   - codes: x*y with one fma remainder correction == RN(x/s) (fp8q_math.h), then the
//     hardware converter, 16 codes = one 16-byte store per lane (the wave writes 1 KB
//     contiguous); the group's first lane writes the scale.
// A flat grid-stride loop over groups handles any m (the pages put M on grid X because
// MoE row counts exceed grid Y's limit; a flat index has no such limit).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8q.h"
#include "fp8q_device.h"
#include "fp8q_launch.h"

#pragma clang fp contract(off)

namespace fp8q {
namespace {

// 512-thread blocks, one 8-group tile per wave (a launch streams the matrix once, in
// order).  Measured on MI355X at 4593 x 5120 and 4593 x 16384 against 256- and 1024-thread
// blocks, two tiles' loads in flight per wave, persistent grids of 4 or 8 blocks per CU and
// non-temporal loads: this form is the fastest or within noise of it at both sizes.
constexpr int kQuantBlock = 512;  // threads per block
constexpr int kGroupsPerWave = 8;
constexpr int kGroupsPerBlock = kGroupsPerWave * (kQuantBlock / 64);

__global__ __launch_bounds__(kQuantBlock) void group_quant_kernel(
    const uint4* __restrict__ x, uint4* __restrict__ q, float* __restrict__ scales,
    int64_t num_groups) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  const int sub = lane & 7;  // lane within its group
  const int64_t wave = (int64_t(blockIdx.x) * kQuantBlock + threadIdx.x) >> 6;
  const int64_t wave_stride = (int64_t(gridDim.x) * kQuantBlock) >> 6;
  for (int64_t base = wave * kGroupsPerWave; base < num_groups;
       base += wave_stride * kGroupsPerWave) {
    const int64_t g = base + (lane >> 3);
    // past the end: re-read the last group (in bounds), nothing is stored for it
    const int64_t gl = g < num_groups ? g : num_groups - 1;
    const uint4 w0 = x[gl * 16 + sub * 2];
    const uint4 w1 = x[gl * 16 + sub * 2 + 1];
    const float amax = max_over_8_lanes(fmaxf(absmax8(w0), absmax8(w1)));
    const float s = group_scale_from_amax(amax);
    const float y = 1.0f / s;  // IEEE division: RN(1/s)
    const uint2 c0 = quant8<true>(w0, s, y);
    const uint2 c1 = quant8<true>(w1, s, y);
    if (g < num_groups) {
      // codes are not read again by this kernel: written with the non-temporal hint
      __builtin_nontemporal_store(v4u{c0.x, c0.y, c1.x, c1.y},
                                  reinterpret_cast<v4u*>(q + g * 8 + sub));
      if (sub == 0) scales[g] = s;
    }
  }
}

// One 256-thread block per 128x128 weight block; edge blocks are clipped to the matrix.
__global__ __launch_bounds__(256) void block_quant_kernel(const uint16_t* __restrict__ w,
                                                          uint8_t* __restrict__ wq,
                                                          float* __restrict__ ws, int n,
                                                          int k, int kblocks) {
  __shared__ float red[4];
  const int nb = blockIdx.y, kb = blockIdx.x;
  const int r0 = nb * 128, c0 = kb * 128;
  const int rows = min(128, n - r0), cols = min(128, k - c0);
  float amax = 0.0f;
  for (int i = threadIdx.x; i < rows * 128; i += 256) {
    int r = i >> 7, c = i & 127;
    if (c < cols) amax = fmaxf(amax, fabsf(bf16_to_f32(w[int64_t(r0 + r) * k + c0 + c])));
  }
  amax = max_over_wave(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float s = group_scale_from_amax(amax);
  const float y = 1.0f / s;
  if (threadIdx.x == 0) ws[int64_t(nb) * kblocks + kb] = s;
  for (int i = threadIdx.x; i < rows * 128; i += 256) {
    int r = i >> 7, c = i & 127;
    if (c < cols) {
      int64_t idx = int64_t(r0 + r) * k + c0 + c;
      float v = div_by_scale(bf16_to_f32(w[idx]), s, y);
      wq[idx] = uint8_t(__builtin_amdgcn_cvt_pk_fp8_f32(clip448(v), 0.0f, 0, false) & 0xFF);
    }
  }
}

__global__ __launch_bounds__(256) void encode_kernel(const float* __restrict__ x,
                                                     uint8_t* __restrict__ q, int64_t n) {
  const int64_t stride = int64_t(gridDim.x) * 256;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride)
    q[i] = uint8_t(__builtin_amdgcn_cvt_pk_fp8_f32(clip448(x[i]), 0.0f, 0, false) & 0xFF);
}

}  // namespace
}  // namespace fp8q

using namespace fp8q;

extern "C" int fp8_group_quant(const uint16_t* x, uint8_t* q, float* scales, int64_t m,
                               int32_t k, hipStream_t stream) {
  if (m < 0 || k <= 0 || k % 128 != 0) return FP8Q_EINVAL;
  if (m > (int64_t(1) << 62) / k) return FP8Q_EINVAL;
  if (m == 0) return FP8Q_OK;
  if (!x || !q || !scales) return FP8Q_ENULL;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scales, 4)) return FP8Q_EALIGN;
  const int64_t groups = m * (k / 128);
  const int64_t blocks = clamp_grid((groups + kGroupsPerBlock - 1) / kGroupsPerBlock);
  launch(group_quant_kernel, dim3(unsigned(blocks)), dim3(kQuantBlock), 0, stream,
         reinterpret_cast<const uint4*>(x), reinterpret_cast<uint4*>(q), scales, groups);
  return launch_status();
}

extern "C" int fp8_block_quant(const uint16_t* w, uint8_t* wq, float* ws, int32_t n,
                               int32_t k, hipStream_t stream) {
  if (n <= 0 || k <= 0) return FP8Q_EINVAL;
  if (!w || !wq || !ws) return FP8Q_ENULL;
  if (!aligned(ws, 4)) return FP8Q_EALIGN;
  const int nblocks = (n + 127) / 128, kblocks = (k + 127) / 128;
  if (nblocks > 65535) return FP8Q_EINVAL;
  launch(block_quant_kernel, dim3(kblocks, nblocks), dim3(256), 0, stream, w,
                     wq, ws, n, k, kblocks);
  return launch_status();
}

extern "C" int fp8_e4m3_encode(const float* x, uint8_t* q, int64_t n, hipStream_t stream) {
  if (n < 0) return FP8Q_EINVAL;
  if (n == 0) return FP8Q_OK;
  if (!x || !q) return FP8Q_ENULL;
  if (!aligned(x, 4)) return FP8Q_EALIGN;
  const int64_t blocks = clamp_grid((n + 255) / 256);
  launch(encode_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream, x, q, n);
  return launch_status();
}
