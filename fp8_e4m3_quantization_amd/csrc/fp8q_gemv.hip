// fp8q_gemv.hip -- the W8A16 decode tier for 1..4 activation rows: bf16 activation times
// E4M3 weight with 128x128 FP32 block scales, FP32 accumulation, bf16 out.
//
// dispatch_proj_decode.rs page: module doc NUMERICS (the W8A16 arithmetic: bf16 activation
// x E4M3 weight with the checkpoint's 128x128 FP32 block scales, which the W8A8 rows
// replace above four rows), DECODE_W8A8_ROWS (four rows or fewer stay on the batch-4 GEMV
// tier, one row on the scalar GEMV: at those widths a GEMV that streams each weight byte
// once is the right shape).
//
// The pages' GEMV tiers are CUDA FFMA loops.  Here the same persistent layout as the W8A8
// decode kernel streams the weights: one 8-wave workgroup per CU walks 16-column output
// strips, wave w owns a fixed 1/8 of the K-groups with its activation fragments held in
// registers for the whole launch, weight slices are prefetched one strip ahead through a
// buffer descriptor, and the 8 partials of each strip meet in LDS once per 4 strips.  Per
// 128-wide group a lane widens its 32 weight codes to bf16 (exact: every E4M3 value is a
// bf16 value) with 16 v_cvt_pk_f32_fp8 and 16 v_perm_b32, and four v_mfma_f32_16x16x32_bf16
// accumulate the group's partial, which the block scale then multiplies in FP32.  The MFMA
// computes 16 activation rows; rows >= m repeat row m-1 and are never stored.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8q.h"
#include "fp8q_device.h"
#include "fp8q_gemm_common.h"
#include "fp8q_launch.h"

#pragma clang fp contract(off)

namespace fp8q {
namespace {

constexpr int kGemvMaxRows = 4;
constexpr int kGemvRound = 4;  // strips per LDS reduction
constexpr int kGemvMaxK = kPWaves * 8 * 128;  // the persistent form holds <= 8 groups per wave

template <int kGpw>
struct GemvSlice {
  v8i b[kGpw];
  float ws[kGpw];
};

// Operand layout (v_mfma_f32_16x16x32_bf16): lane l supplies row (l & 15) and 8 values of
// k.  For group g the lane holds k = 128g + 32*(l>>4) + [0, 32) of its row (activation
// row for A, weight row = output column for B); MFMA i of the group uses the 8 values at
// +8i.  A and B use the same assignment, so the four MFMAs sum every k of the group once.
// Accumulator: lane l, register j holds activation row 4*(l>>4) + j, column l & 15; with
// m <= 4 only lanes 0..15 carry stored rows.
template <int kGpw>
__global__ __launch_bounds__(64 * kPWaves) void w8a16_persistent_kernel(
    const uint16_t* __restrict__ a, ProjSet ps, int m, int k, int total_strips, int half_from) {
  __shared__ float s_part[2][kGemvRound * kPWaves * 64];
  __shared__ uint4 s_tile[kPWaves * ActTile<16>::kUints];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int groups = k >> 7;
  const int g0 = (groups * wv) / kPWaves;
  const int cnt = (groups * (wv + 1)) / kPWaves - g0;  // 0 <= cnt <= kGpw
  const int row = lane & 15, koff = (lane >> 4) * 32;
  int goff[kGpw];  // first k of slice group u (a short slice repeats its last group; the
                   // repeat is skipped in the multiply)
#pragma unroll
  for (int u = 0; u < kGpw; ++u) goff[u] = (g0 + max(0, min(u, cnt - 1))) * 128;

  const int total_items = item_count(total_strips, half_from);  // see StripItem
  auto fetch = [&](int s, GemvSlice<kGpw>& sl) {
    const bool valid = s < total_items;
    const StripItem it = strip_item(valid ? s : total_items - 1, half_from);
    int p, n0;
    locate_strip(ps, it.strip, &p, &n0);
    const __amdgpu_buffer_rsrc_t r =
        make_strip_rsrc(ps.w[p] + int64_t(n0 + it.col0) * k, k, valid, it.cols);
    const_float* wsp = (const_float*)(ps.ws[p] + int64_t(n0 >> 7) * groups);
#pragma unroll
    for (int u = 0; u < kGpw; ++u) sl.b[u] = buffer_load32<0>(r, row * k + koff + goff[u]);
#pragma unroll
    for (int u = 0; u < kGpw; ++u) sl.ws[u] = wsp[goff[u] >> 7];
  };

  const int stride = int(gridDim.x);
  const int first = first_strip(int(blockIdx.x), stride);
  const int nit = (total_items - first + stride - 1) / stride;
  if (nit <= 0) return;

  // activation tiles first, then the first weight prefetch, then the fragments (through
  // LDS, see ActTile; they stay in registers for the whole launch)
  using Tile = ActTile<16>;
  v4u stage[kGpw][Tile::kLoads];
  const uint8_t* ab = reinterpret_cast<const uint8_t*>(a);
#pragma unroll
  for (int u = 0; u < kGpw; ++u) Tile::load(ab + 2 * goff[u], 2 * int64_t(k), m, lane, stage[u]);
  GemvSlice<kGpw> buf[2];
  uint4 af[kGpw][4];
  auto exchange_all = [&]() {
#pragma unroll
    for (int u = 0; u < kGpw; ++u)
      Tile::exchange(s_tile + wv * Tile::kUints, stage[u], lane, koff >> 3, af[u]);
  };
  if constexpr (kGpw <= 6) {
    fetch(first, buf[0]);
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the fragment exchange
    exchange_all();
  } else {  // staged tiles, fragments and a prefetched slice would not fit in registers
    exchange_all();
    fetch(first, buf[0]);
  }

  auto multiply = [&](const GemvSlice<kGpw>& cur) {
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < kGpw; ++u) {
      if (u < cnt) {  // wave-uniform
        v4f c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(v8bf16, af[u][i]),
              widen8(uint32_t(cur.b[u][2 * i]), uint32_t(cur.b[u][2 * i + 1])), c, 0, 0, 0);
        const float w = cur.ws[u];
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] = __builtin_fmaf(c[q], w, acc[q]);
      }
    }
    return acc;
  };

  int par = 0;
  for (int i = 0; i < nit; i += kGemvRound) {
    float* part = s_part[par];  // [round strip][wave][register][16 columns]
#pragma unroll
    for (int j = 0; j < kGemvRound; ++j) {
      fetch(first + (i + j + 1) * stride, buf[(j + 1) & 1]);
      if (i + j < nit) {
        const v4f acc = multiply(buf[j & 1]);
        if (lane < 16) {
#pragma unroll
          for (int q = 0; q < 4; ++q) part[((j * kPWaves + wv) * 4 + q) * 16 + lane] = acc[q];
        }
      }
    }
    lds_barrier();
    // Reduce: thread t < 256 owns output (round strip t/64, register (t/16)%4, column t%16).
    // Every LDS read of the round comes before its one store.
    const int t = int(threadIdx.x);
    if (t < kGemvRound * 64) {
      const int j = t >> 6, q = (t >> 4) & 3, c = t & 15;
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < kPWaves; ++w) sum += part[((j * kPWaves + w) * 4 + q) * 16 + c];
      if (i + j < nit && q < m) {
        const StripItem it = strip_item(first + (i + j) * stride, half_from);
        int p, n0;
        locate_strip(ps, it.strip, &p, &n0);
        if (c < it.cols) ps.out[p][int64_t(q) * ps.ldc[p] + n0 + it.col0 + c] = f32_to_bf16_rne(sum);
      }
    }
    par ^= 1;
  }
}

// Long-K form (k > 8192): one 8-wave workgroup per 16-column strip; wave w walks a
// contiguous 1/8 of the K-groups kChunk at a time (weights through the strip's buffer
// descriptor, activation fragments from L2), then the 8 partials meet in LDS.  Same
// operand layout and per-group arithmetic as the persistent kernel.
constexpr int kGemvLongChunk = 4;
constexpr int kGemvLongMaxK = 131072;

__global__ __launch_bounds__(64 * kPWaves) void w8a16_long_kernel(const uint16_t* __restrict__ a,
                                                                  ProjSet ps, int m, int k) {
  __shared__ float s_part[kPWaves * 64];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int groups = k >> 7;
  int p, n0;
  locate_strip(ps, int(blockIdx.x), &p, &n0);
  const __amdgpu_buffer_rsrc_t r = make_strip_rsrc(ps.w[p] + int64_t(n0) * k, k, true);
  const_float* wsp = (const_float*)(ps.ws[p] + int64_t(n0 >> 7) * groups);
  const int row = lane & 15, koff = (lane >> 4) * 32;
  const int arow = row < m ? row : m - 1;
  const uint4* ap = reinterpret_cast<const uint4*>(a + int64_t(arow) * k + koff);
  const int g_begin = (groups * wv) / kPWaves, g_end = (groups * (wv + 1)) / kPWaves;

  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int g = g_begin; g < g_end; g += kGemvLongChunk) {
    v8i wb[kGemvLongChunk];
    uint4 af[kGemvLongChunk][4];
    float ws[kGemvLongChunk];
#pragma unroll
    for (int u = 0; u < kGemvLongChunk; ++u) {
      const int gu = min(g + u, g_end - 1);  // a short chunk re-reads its last group
      wb[u] = buffer_load32<0>(r, row * k + koff + gu * 128);
#pragma unroll
      for (int i = 0; i < 4; ++i) af[u][i] = ap[gu * 16 + i];
      ws[u] = wsp[gu];
    }
#pragma unroll
    for (int u = 0; u < kGemvLongChunk; ++u) {
      if (g + u < g_end) {  // wave-uniform
        v4f c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(v8bf16, af[u][i]),
              widen8(uint32_t(wb[u][2 * i]), uint32_t(wb[u][2 * i + 1])), c, 0, 0, 0);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[q] = __builtin_fmaf(c[q], ws[u], acc[q]);
      }
    }
  }
  // partials of lanes 0..15 (the stored rows) meet in LDS; fixed summation order
  if (lane < 16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) s_part[(wv * 4 + q) * 16 + lane] = acc[q];
  }
  __syncthreads();
  const int t = int(threadIdx.x);
  if (t < 64) {
    const int q = t >> 4, c = t & 15;
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < kPWaves; ++w) sum += s_part[(w * 4 + q) * 16 + c];
    if (q < m) ps.out[p][int64_t(q) * ps.ldc[p] + n0 + c] = f32_to_bf16_rne(sum);
  }
}

template <int kGpw>
int launch_gemv(const uint16_t* a, const ProjSet& ps, int m, int k, int total,
                hipStream_t stream) {
  const int grid = total < num_cus() ? total : num_cus();
  launch(w8a16_persistent_kernel<kGpw>, dim3(grid), dim3(64 * kPWaves), 0, stream, a, ps, m,
         k, total, halved_from(total, grid));
  return launch_status();
}

int run_gemv(const uint16_t* a, const ProjSet& ps, int m, int k, hipStream_t stream) {
  const int total = ps.strip_end[ps.count - 1];
  // k a multiple of 1024: the weight stream staged through LDS in whole 1 KB rows (the W8A8
  // decode GEMM's staged form with a bf16 activation)
  if (k % 1024 == 0 && k <= kGemvMaxK) return run_w8a16_staged(a, ps, m, k, stream);
  if (k > kGemvMaxK) {
    launch(w8a16_long_kernel, dim3(unsigned(total)), dim3(64 * kPWaves), 0, stream, a, ps, m, k);
    return launch_status();
  }
  switch ((k / 128 + kPWaves - 1) / kPWaves) {
    case 1: return launch_gemv<1>(a, ps, m, k, total, stream);
    case 2: return launch_gemv<2>(a, ps, m, k, total, stream);
    case 3: return launch_gemv<3>(a, ps, m, k, total, stream);
    case 4: return launch_gemv<4>(a, ps, m, k, total, stream);
    case 5: return launch_gemv<5>(a, ps, m, k, total, stream);
    case 6: return launch_gemv<6>(a, ps, m, k, total, stream);
    case 7: return launch_gemv<7>(a, ps, m, k, total, stream);
    case 8: return launch_gemv<8>(a, ps, m, k, total, stream);
    default: return FP8Q_EINVAL;
  }
}

int check_gemv_proj(const uint8_t* w_q, const float* w_scale, const uint16_t* out, int32_t n,
                    int32_t ldc) {
  if (n <= 0 || n % 128 != 0 || ldc < n) return FP8Q_EINVAL;
  if (!w_q || !w_scale || !out) return FP8Q_ENULL;
  if (!aligned(w_q, 16) || !aligned(w_scale, 4) || !aligned(out, 2)) return FP8Q_EALIGN;
  return FP8Q_OK;
}

}  // namespace
}  // namespace fp8q

using namespace fp8q;

extern "C" int w8a16_block_gemv_grouped(const uint16_t* a, const fp8q_gemm_proj* projs,
                                        int32_t count, int32_t m, int32_t k,
                                        hipStream_t stream) {
  if (count < 1 || count > kMaxProj) return FP8Q_EINVAL;
  if (m < 1 || m > kGemvMaxRows || k <= 0 || k % 128 != 0 || k > kGemvLongMaxK)
    return FP8Q_EINVAL;
  if (!a || !projs) return FP8Q_ENULL;
  if (!aligned(a, 16)) return FP8Q_EALIGN;
  ProjSet ps = {};
  int64_t end = 0;
  for (int p = 0; p < count; ++p) {
    const int rc = check_gemv_proj(projs[p].w_q, projs[p].w_scale, projs[p].out, projs[p].n,
                                   projs[p].ldc);
    if (rc != FP8Q_OK) return rc;
    end += projs[p].n / 16;
    if (end > 0x7FFFFFFF) return FP8Q_EINVAL;
    ps.w[p] = projs[p].w_q;
    ps.ws[p] = projs[p].w_scale;
    ps.out[p] = projs[p].out;
    ps.ldc[p] = projs[p].ldc;
    ps.strip_end[p] = int(end);
  }
  ps.count = count;
  return run_gemv(a, ps, m, k, stream);
}

extern "C" int w8a16_block_gemv(const uint16_t* a, const uint8_t* w_q, const float* w_scale,
                                uint16_t* out, int32_t m, int32_t n, int32_t k, int32_t ldc,
                                hipStream_t stream) {
  const fp8q_gemm_proj p = {w_q, w_scale, out, n, ldc};
  return w8a16_block_gemv_grouped(a, &p, 1, m, k, stream);
}
