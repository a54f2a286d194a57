// fp8q_gemm.hip -- block-scaled W8A8 GEMM for decode widths (1..16 activation rows).
//
// dispatch_proj_decode.rs page: module doc NUMERICS (E4M3 activations with per-token
// 1x128 FP32 scales times E4M3 weights with 128x128 FP32 block scales, FP32 epilogue),
// decode_w8a8_gemm (out = act_fp8 @ weight^T at row pitch ldc), DecodeW8a8Plan /
// decode_w8a8_selected (n % 128, k % 128, ldc >= n), DECODE_W8A8_ROWS (<= 16 rows).
//
// At <= 16 rows the op is a stream over the N*K weight bytes (2*16 flop per byte against
// a machine balance in the hundreds), so the kernel is built to keep HBM busy:
//   - one gfx950 MFMA v_mfma_f32_16x16x128_f8f6f4 covers exactly one 128-wide K-group of
//     a 16(rows) x 16(columns) tile, so the block scales apply per instruction: the
//     partial of group g is scaled by a_scale[r,g] * w_scale[c/128,g] and added in FP32;
//   - a workgroup owns 16 output columns; its waves split K and each streams its slice
//     of the 16 weight rows with 16-byte loads, a chunk of groups in flight at a time;
//   - the activation (<= 16 x K bytes, L2-resident) is read per wave; its scales are
//     staged once per workgroup in LDS, transposed to [group][row];
//   - the K-split partials are summed in LDS and written once as bf16 (RNE).
// Rows >= m are fed zeros and never stored, so only (m-1)*ldc + n elements are written.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8q.h"
#include "fp8q_device.h"
#include "fp8q_launch.h"

#pragma clang fp contract(off)

namespace fp8q {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kMaxGemmK = 131072;  // LDS holds the [k/128][16] activation scales

__device__ __forceinline__ v8i load32(const uint8_t* p) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  uint4 a = q[0], b = q[1];
  v8i r;
  r[0] = int(a.x); r[1] = int(a.y); r[2] = int(a.z); r[3] = int(a.w);
  r[4] = int(b.x); r[5] = int(b.y); r[6] = int(b.z); r[7] = int(b.w);
  return r;
}

// E4M3 x E4M3 -> FP32, one 16x16 tile over one 128-wide K-group (no scaling).
__device__ __forceinline__ v4f mfma_group(v8i a, v8i b) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  // format 0 = E4M3 for both operands; zero scale operands select the unscaled MFMA
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

template <int kWaves, int kChunk>
__global__ __launch_bounds__(64 * kWaves) void w8a8_gemm_kernel(
    const uint8_t* __restrict__ a_q, const float* __restrict__ a_scale,
    const uint8_t* __restrict__ w_q, const float* __restrict__ w_scale,
    uint16_t* __restrict__ out, int m, int k, int ldc) {
  extern __shared__ float smem[];
  const int groups = k >> 7;
  float* s_as = smem;                    // [groups][16]
  float* s_part = smem + groups * 16;    // [kWaves][4][64]
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n0 = blockIdx.x * 16;

  for (int i = tid; i < groups * 16; i += 64 * kWaves) {
    const int g = i >> 4, r = i & 15;
    s_as[i] = r < m ? a_scale[int64_t(r) * groups + g] : 0.0f;
  }
  __syncthreads();

  // Operand layout: lane l supplies row (l & 15) of the 16-row operand and bytes
  // [32*(l>>4), 32*(l>>4)+32) of the group; A (activation rows) and B (weight rows,
  // i.e. output columns) use the same byte->k assignment, so the sum over k is exact
  // whatever order the instruction walks it in.
  const int row = lane & 15;
  const int koff = (lane >> 4) * 32;
  const uint8_t* wp = w_q + int64_t(n0 + row) * k + koff;
  const bool a_live = row < m;
  const uint8_t* ap = a_q + int64_t(a_live ? row : 0) * k + koff;
  const float* wsp = w_scale + int64_t(n0 >> 7) * groups;
  const float* asp = s_as + (lane >> 4) * 4;  // the 4 output rows this lane holds

  const int g_begin = (groups * wv) / kWaves;
  const int g_end = (groups * (wv + 1)) / kWaves;
  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const v8i zero8 = {0, 0, 0, 0, 0, 0, 0, 0};

  int g = g_begin;
  for (; g + kChunk <= g_end; g += kChunk) {
    v8i b[kChunk], a[kChunk];
#pragma unroll
    for (int u = 0; u < kChunk; ++u) b[u] = load32(wp + int64_t(g + u) * 128);
#pragma unroll
    for (int u = 0; u < kChunk; ++u) a[u] = a_live ? load32(ap + int64_t(g + u) * 128) : zero8;
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const v4f c = mfma_group(a[u], b[u]);
      const float ws = wsp[g + u];
      const float4 as = *reinterpret_cast<const float4*>(asp + (g + u) * 16);
      acc[0] = __builtin_fmaf(c[0], as.x * ws, acc[0]);
      acc[1] = __builtin_fmaf(c[1], as.y * ws, acc[1]);
      acc[2] = __builtin_fmaf(c[2], as.z * ws, acc[2]);
      acc[3] = __builtin_fmaf(c[3], as.w * ws, acc[3]);
    }
  }
  for (; g < g_end; ++g) {
    const v8i b = load32(wp + int64_t(g) * 128);
    const v8i a = a_live ? load32(ap + int64_t(g) * 128) : zero8;
    const v4f c = mfma_group(a, b);
    const float ws = wsp[g];
    const float4 as = *reinterpret_cast<const float4*>(asp + g * 16);
    acc[0] = __builtin_fmaf(c[0], as.x * ws, acc[0]);
    acc[1] = __builtin_fmaf(c[1], as.y * ws, acc[1]);
    acc[2] = __builtin_fmaf(c[2], as.z * ws, acc[2]);
    acc[3] = __builtin_fmaf(c[3], as.w * ws, acc[3]);
  }

  // Accumulator layout: lane l, register j holds row 4*(l>>4) + j, column l & 15.
#pragma unroll
  for (int j = 0; j < 4; ++j) s_part[(wv * 4 + j) * 64 + lane] = acc[j];
  __syncthreads();
  for (int t = tid; t < 256; t += 64 * kWaves) {
    const int j = t >> 6, l = t & 63;
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) sum += s_part[(w * 4 + j) * 64 + l];
    const int r = 4 * (l >> 4) + j, c = l & 15;
    if (r < m) out[int64_t(r) * ldc + n0 + c] = f32_to_bf16_rne(sum);
  }
}

template <int kWaves, int kChunk>
int launch_gemm(const uint8_t* a_q, const float* a_scale, const uint8_t* w_q,
                const float* w_scale, uint16_t* out, int m, int n, int k, int ldc,
                hipStream_t stream) {
  const size_t lds = size_t(k / 128) * 16 * sizeof(float) + size_t(kWaves) * 256 * sizeof(float);
  hipLaunchKernelGGL((w8a8_gemm_kernel<kWaves, kChunk>), dim3(n / 16), dim3(64 * kWaves),
                     lds, stream, a_q, a_scale, w_q, w_scale, out, m, k, ldc);
  return launch_status();
}

}  // namespace
}  // namespace fp8q

using namespace fp8q;

extern "C" int w8a8_block_gemm(const uint8_t* a_q, const float* a_scale, const uint8_t* w_q,
                               const float* w_scale, uint16_t* out, int32_t m, int32_t n,
                               int32_t k, int32_t ldc, hipStream_t stream) {
  if (m < 1 || m > 16 || n <= 0 || n % 128 != 0 || k <= 0 || k % 128 != 0 || ldc < n ||
      k > kMaxGemmK)
    return FP8Q_EINVAL;
  if (!a_q || !a_scale || !w_q || !w_scale || !out) return FP8Q_ENULL;
  if (!aligned(a_q, 16) || !aligned(w_q, 16) || !aligned(a_scale, 4) ||
      !aligned(w_scale, 4) || !aligned(out, 2))
    return FP8Q_EALIGN;
  return launch_gemm<4, 5>(a_q, a_scale, w_q, w_scale, out, m, n, k, ldc, stream);
}
