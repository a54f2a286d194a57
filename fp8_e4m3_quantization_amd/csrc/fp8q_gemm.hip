// fp8q_gemm.hip -- block-scaled W8A8 GEMM for decode widths (1..16 activation rows).
//
// dispatch_proj_decode.rs page: module doc NUMERICS (E4M3 activations with per-token
// 1x128 FP32 scales times E4M3 weights with 128x128 FP32 block scales, FP32 epilogue),
// decode_w8a8_gemm (out = act_fp8 @ weight^T at row pitch ldc), DecodeW8a8Plan /
// decode_w8a8_selected (n % 128, k % 128, ldc >= n), DECODE_W8A8_ROWS (<= 16 rows).
//
// At <= 16 rows the op is a stream over the N*K weight bytes (2*16 flop per byte against
// a machine balance in the hundreds), so the kernels are built to keep HBM busy:
//   - one gfx950 MFMA v_mfma_f32_16x16x128_f8f6f4 covers exactly one 128-wide K-group of
//     a 16(rows) x 16(columns) tile, so the block scales apply per instruction: the
//     partial of group g is scaled by a_scale[r,g] * w_scale[c/128,g] and added in FP32;
//   - the work unit is a strip of 16 output columns; the waves of a workgroup split K and
//     each streams its slice of the strip's 16 weight rows with 16-byte loads;
//   - the K-split partials are summed in LDS and written once as bf16 (RNE).
// Two forms: the persistent kernel below (k <= 8192; one workgroup per CU walks strips,
// each wave keeping its activation slice in registers), and w8a8_gemm_kernel for longer k
// (one workgroup per strip; the activation, <= 16 x K bytes and L2-resident, is read per
// wave and its scales are staged in LDS, transposed to [group][row]).
// Rows >= m are fed zeros and never stored, so only (m-1)*ldc + n elements are written.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8q.h"
#include "fp8q_device.h"
#include "fp8q_gemm_common.h"
#include "fp8q_launch.h"

#pragma clang fp contract(off)

namespace fp8q {
namespace {

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

// ---------------------------------------------------------------------------------
// Persistent form: one 8-wave workgroup per CU walks output strips of 16 columns.
// Wave w owns a fixed slice of K-groups: its activation fragments and scales for that
// slice are loaded once (the tiles through LDS, see ActTile) and stay in registers for the
// whole kernel, so the only global traffic in the strip loop is the weight stream.  Each
// wave prefetches the next strip's weight slice while it multiplies the current one; the
// 8 K-slice partials of a strip meet in LDS (double-buffered, one barrier per round of
// strips, below) and one pass writes bf16.  Several projections that read the same
// activation can share one launch: strips are numbered across them, and each block walks
// them from first_strip (adjacent strips on one XCD).
// Weight loads go through a buffer descriptor per strip (make_strip_rsrc); the cache
// policy bits of those loads:
#ifndef FP8Q_GEMM_AUX
#define FP8Q_GEMM_AUX 0
#endif
#ifndef FP8Q_GEMM_NT_OUT
#define FP8Q_GEMM_NT_OUT 0  // 1: bf16 outputs written with the non-temporal hint
#endif

template <int kGpw>
struct Slice {
  v8i b[kGpw];
  float ws[kGpw];
};

// Strips are processed in rounds of kRound: a wave multiplies its K-slice of kRound strips
// back to back (its partial tiles stay in registers), then all waves meet once -- partials
// to LDS, one barrier, a fixed-order sum over the waves, bf16 stores.  Per-strip barriers
// would tie every strip to the slowest wave's load latency.  The LDS partial area is
// double-buffered across rounds, so one barrier per round suffices.
// Where the activation comes from: already quantized (codes + token-major scales), or
// bf16, quantized by the GEMM itself (each wave quantizes its own K-slice in registers
// with the group quantizer's arithmetic, so the codes are bit-identical to
// fp8_group_quant's; optionally they are written out, each workgroup a share).
struct ActSrc {
  const uint8_t* a_q;
  const float* a_scale;
  const uint16_t* a_bf16;
  uint8_t* q_out;
  float* s_out;
};

template <int kGpw, int kDepth, int kAux, int kRound, bool kQuant>
__global__ __launch_bounds__(64 * kPWaves) void w8a8_persistent_kernel(
    ActSrc act, ProjSet ps, int m, int k, int total_strips) {
  static_assert(kRound % (kDepth + 1) == 0, "buffer index must be static within a round");
  static_assert(kRound * 256 == kPWaves * 64 * 2, "reduce: two outputs per lane");
  __shared__ float s_part[2][kRound * kPWaves * 4 * 64];
  __shared__ uint4 s_tile[kPWaves * ActTile<kQuant ? 16 : 8>::kUints];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int groups = k >> 7;
  const int g0 = (groups * wv) / kPWaves;
  const int cnt = (groups * (wv + 1)) / kPWaves - g0;  // 0 <= cnt <= kGpw
  const int row = lane & 15, koff = (lane >> 4) * 32;
  int goff[kGpw];  // first k of slice group u (a short slice re-reads its last group,
                   // whose activation fragment below is zero)
#pragma unroll
  for (int u = 0; u < kGpw; ++u) goff[u] = (g0 + max(0, min(u, cnt - 1))) * 128;

  auto fetch = [&](int s, Slice<kGpw>& sl) {
    const bool valid = s < total_strips;
    int p, n0;
    locate_strip(ps, valid ? s : total_strips - 1, &p, &n0);
    const __amdgpu_buffer_rsrc_t r = make_strip_rsrc(ps.w[p] + int64_t(n0) * k, k, valid);
    const_float* wsp = (const_float*)(ps.ws[p] + int64_t(n0 >> 7) * groups);
#pragma unroll
    for (int u = 0; u < kGpw; ++u) sl.b[u] = buffer_load32<kAux>(r, row * k + koff + goff[u]);
#pragma unroll
    for (int u = 0; u < kGpw; ++u) sl.ws[u] = wsp[goff[u] >> 7];
  };

  const int stride = int(gridDim.x);
  const int first = first_strip(int(blockIdx.x), stride);
  const int nit = (total_strips - first + stride - 1) / stride;
  if (nit <= 0) return;

  // 1) raw activation loads, 2) the first weight prefetch, 3) activation fragments: the
  // fragments wait only for the loads issued before the prefetch, so the weight stream
  // starts without waiting for the activation (load counters retire in order).  The
  // activation tiles reach the fragments through LDS (ActTile).
  using Tile = ActTile<kQuant ? 16 : 8>;
  uint4* tile = s_tile + wv * Tile::kUints;
  v8i a[kGpw];
  float4 as[kGpw];
  float scv[kGpw];  // kQuant: this lane's row scale of each slice group
  Slice<kGpw> buf[kDepth + 1];
  const v8i zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
  const int r0 = 4 * (lane >> 4);
  if constexpr (!kQuant) {
    v4u raw[kGpw][Tile::kLoads];
    float4 rs[kGpw];
#pragma unroll
    for (int u = 0; u < kGpw; ++u) {
      Tile::load(act.a_q + goff[u], k, m, lane, raw[u]);
      const int g = goff[u] >> 7;
      rs[u].x = act.a_scale[int64_t(min(r0 + 0, m - 1)) * groups + g];
      rs[u].y = act.a_scale[int64_t(min(r0 + 1, m - 1)) * groups + g];
      rs[u].z = act.a_scale[int64_t(min(r0 + 2, m - 1)) * groups + g];
      rs[u].w = act.a_scale[int64_t(min(r0 + 3, m - 1)) * groups + g];
    }
#pragma unroll
    for (int j = 0; j < kDepth; ++j) fetch(first + j * stride, buf[j]);
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the activation math
#pragma unroll
    for (int u = 0; u < kGpw; ++u) {
      const bool live = u < cnt;
      uint4 f[2];
      Tile::exchange(tile, raw[u], lane, koff >> 4, f);
      const v8i fr = {int(f[0].x), int(f[0].y), int(f[0].z), int(f[0].w),
                      int(f[1].x), int(f[1].y), int(f[1].z), int(f[1].w)};
      a[u] = (live && row < m) ? fr : zero8;
      as[u].x = (live && r0 + 0 < m) ? rs[u].x : 0.0f;
      as[u].y = (live && r0 + 1 < m) ? rs[u].y : 0.0f;
      as[u].z = (live && r0 + 2 < m) ? rs[u].z : 0.0f;
      as[u].w = (live && r0 + 3 < m) ? rs[u].w : 0.0f;
    }
  } else {
    // lane l gets elements [32*(l>>4), +32) of row (l & 15) in each slice group: the four
    // lanes l, l^16, l^32, l^48 together hold the row's 128-element group
    v4u stage[kGpw][Tile::kLoads];
    const uint8_t* xb = reinterpret_cast<const uint8_t*>(act.a_bf16);
#pragma unroll
    for (int u = 0; u < kGpw; ++u) Tile::load(xb + 2 * goff[u], 2 * int64_t(k), m, lane, stage[u]);
#pragma unroll
    for (int j = 0; j < kDepth; ++j) fetch(first + j * stride, buf[j]);
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the activation math
#pragma unroll
    for (int u = 0; u < kGpw; ++u) {
      const bool live = u < cnt;
      uint4 raw[4];
      Tile::exchange(tile, stage[u], lane, koff >> 3, raw);
      float amax = fmaxf(fmaxf(absmax8(raw[0]), absmax8(raw[1])),
                         fmaxf(absmax8(raw[2]), absmax8(raw[3])));
      amax = fmaxf(amax, __shfl_xor(amax, 16));
      amax = fmaxf(amax, __shfl_xor(amax, 32));
      const float sc = group_scale_from_amax(amax);
      const float y = 1.0f / sc;  // IEEE division: RN(1/s)
      const uint2 c0 = quant8<true>(raw[0], sc, y), c1 = quant8<true>(raw[1], sc, y);
      const uint2 c2 = quant8<true>(raw[2], sc, y), c3 = quant8<true>(raw[3], sc, y);
      v8i f;
      f[0] = int(c0.x); f[1] = int(c0.y); f[2] = int(c1.x); f[3] = int(c1.y);
      f[4] = int(c2.x); f[5] = int(c2.y); f[6] = int(c3.x); f[7] = int(c3.y);
      a[u] = (live && row < m) ? f : zero8;
      // row r's scale sits in lane r (and r+16, r+32, r+48)
      const float s0 = __shfl(sc, r0 + 0), s1 = __shfl(sc, r0 + 1);
      const float s2 = __shfl(sc, r0 + 2), s3 = __shfl(sc, r0 + 3);
      as[u].x = (live && r0 + 0 < m) ? s0 : 0.0f;
      as[u].y = (live && r0 + 1 < m) ? s1 : 0.0f;
      as[u].z = (live && r0 + 2 < m) ? s2 : 0.0f;
      as[u].w = (live && r0 + 3 < m) ? s3 : 0.0f;
      scv[u] = sc;
    }
  }

  // Optional code/scale output of the fused quantization.  Every workgroup holds every code
  // (a[u] of the lanes of row (l & 15)), so the (row, group) tiles are dealt round robin
  // over the workgroups and each writes its share.  The stores go out in the last round,
  // after its fetches and multiplies are issued: stores retire through the same in-order
  // counter as loads, so any strip waited for after them would wait for them too.
  auto write_codes = [&]() {
#pragma unroll
    for (int u = 0; u < kGpw; ++u) {
      const int g = goff[u] >> 7;
      if (u < cnt && row < m && (row * groups + g) % stride == int(blockIdx.x)) {
        uint4* qo = reinterpret_cast<uint4*>(act.q_out + int64_t(row) * k + goff[u] + koff);
        qo[0] = make_uint4(uint32_t(a[u][0]), uint32_t(a[u][1]), uint32_t(a[u][2]), uint32_t(a[u][3]));
        qo[1] = make_uint4(uint32_t(a[u][4]), uint32_t(a[u][5]), uint32_t(a[u][6]), uint32_t(a[u][7]));
        if (lane < 16) act.s_out[int64_t(row) * groups + g] = scv[u];
      }
    }
  };

  auto multiply = [&](const Slice<kGpw>& cur) {
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < kGpw; ++u) {
      const v4f c = mfma_group(a[u], cur.b[u]);
      const float w = cur.ws[u];
      acc[0] = __builtin_fmaf(c[0], as[u].x * w, acc[0]);
      acc[1] = __builtin_fmaf(c[1], as[u].y * w, acc[1]);
      acc[2] = __builtin_fmaf(c[2], as[u].z * w, acc[2]);
      acc[3] = __builtin_fmaf(c[3], as[u].w * w, acc[3]);
    }
    return acc;
  };

  // this workgroup's strips: first + i * stride for i < nit; kDepth ahead in flight
  int par = 0;
  for (int i = 0; i < nit; i += kRound) {
    float* part = s_part[par];  // [round strip][wave][4][64]
#pragma unroll
    for (int j = 0; j < kRound; ++j) {
      fetch(first + (i + j + kDepth) * stride, buf[(j + kDepth) % (kDepth + 1)]);
      if (i + j < nit) {
        const v4f acc = multiply(buf[j % (kDepth + 1)]);
#pragma unroll
        for (int q = 0; q < 4; ++q) part[((j * kPWaves + wv) * 4 + q) * 64 + lane] = acc[q];
      }
    }
    if constexpr (kQuant) {
      if (i + kRound >= nit && act.q_out != nullptr) write_codes();  // the last round
    }
    lds_barrier();
    // Reduce: wave w owns half of round strip w/2 (128 of its 256 outputs, 2 per lane).
    // All LDS reads come before the two stores: a store retires through the same in-order
    // counter as the prefetch loads, so nothing after a store may wait on that counter.
    {
      const int j = wv >> 1;                  // wave-uniform
      const int q0 = (wv & 1) * 2;
      float sum[2] = {0.0f, 0.0f};
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int w = 0; w < kPWaves; ++w) sum[x] += part[((j * kPWaves + w) * 4 + q0 + x) * 64 + lane];
      if (i + j < nit) {
        int p, n0;
        locate_strip(ps, first + (i + j) * stride, &p, &n0);
        uint16_t* o = ps.out[p] + n0 + (lane & 15);
        const int ldc = ps.ldc[p];
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const int r = 4 * (lane >> 4) + q0 + x;
#if FP8Q_GEMM_NT_OUT
          if (r < m) __builtin_nontemporal_store(f32_to_bf16_rne(sum[x]), o + int64_t(r) * ldc);
#else
          if (r < m) o[int64_t(r) * ldc] = f32_to_bf16_rne(sum[x]);
#endif
        }
      }
    }
    par ^= 1;
  }
}

template <int kWaves, int kChunk>
int launch_gemm(const uint8_t* a_q, const float* a_scale, const uint8_t* w_q,
                const float* w_scale, uint16_t* out, int m, int n, int k, int ldc,
                hipStream_t stream) {
  const size_t lds = size_t(k / 128) * 16 * sizeof(float) + size_t(kWaves) * 256 * sizeof(float);
  launch((w8a8_gemm_kernel<kWaves, kChunk>), dim3(n / 16), dim3(64 * kWaves),
                     lds, stream, a_q, a_scale, w_q, w_scale, out, m, k, ldc);
  return launch_status();
}

template <int kGpw, bool kQuant>
int launch_persistent(const ActSrc& act, const ProjSet& ps, int m, int k, int total,
                      hipStream_t stream) {
  const int grid = total < num_cus() ? total : num_cus();
  constexpr int kDepth = 1;
  constexpr int kRound = 4;
  launch((w8a8_persistent_kernel<kGpw, kDepth, FP8Q_GEMM_AUX, kRound, kQuant>), dim3(grid),
         dim3(64 * kPWaves), 0, stream, act, ps, m, k, total);
  return launch_status();
}

// Persistent kernel for k <= 8 * 8 * 128 (each wave holds at most 8 groups).
template <bool kQuant>
int run_persistent(const ActSrc& act, const ProjSet& ps, int m, int k, hipStream_t stream) {
  const int total = ps.strip_end[ps.count - 1];
  const int gpw = (k / 128 + kPWaves - 1) / kPWaves;
  switch (gpw) {
    case 1: return launch_persistent<1, kQuant>(act, ps, m, k, total, stream);
    case 2: return launch_persistent<2, kQuant>(act, ps, m, k, total, stream);
    case 3: return launch_persistent<3, kQuant>(act, ps, m, k, total, stream);
    case 4: return launch_persistent<4, kQuant>(act, ps, m, k, total, stream);
    case 5: return launch_persistent<5, kQuant>(act, ps, m, k, total, stream);
    case 6: return launch_persistent<6, kQuant>(act, ps, m, k, total, stream);
    case 7: return launch_persistent<7, kQuant>(act, ps, m, k, total, stream);
    case 8: return launch_persistent<8, kQuant>(act, ps, m, k, total, stream);
    default: return FP8Q_EINVAL;
  }
}

constexpr int kPersistentMaxK = kPWaves * 8 * 128;

}  // namespace
}  // namespace fp8q

using namespace fp8q;

namespace {
int check_gemm_common(const uint8_t* a_q, const float* a_scale, int32_t m, int32_t k) {
  if (m < 1 || m > 16 || k <= 0 || k % 128 != 0 || k > kMaxGemmK) return FP8Q_EINVAL;
  if (!a_q || !a_scale) return FP8Q_ENULL;
  if (!aligned(a_q, 16) || !aligned(a_scale, 4)) return FP8Q_EALIGN;
  return FP8Q_OK;
}

int check_proj(const uint8_t* w_q, const float* w_scale, const uint16_t* out, int32_t n,
               int32_t ldc) {
  if (n <= 0 || n % 128 != 0 || ldc < n) return FP8Q_EINVAL;
  if (!w_q || !w_scale || !out) return FP8Q_ENULL;
  if (!aligned(w_q, 16) || !aligned(w_scale, 4) || !aligned(out, 2)) return FP8Q_EALIGN;
  return FP8Q_OK;
}
}  // namespace

extern "C" int w8a8_block_gemm(const uint8_t* a_q, const float* a_scale, const uint8_t* w_q,
                               const float* w_scale, uint16_t* out, int32_t m, int32_t n,
                               int32_t k, int32_t ldc, hipStream_t stream) {
  int rc = check_gemm_common(a_q, a_scale, m, k);
  if (rc == FP8Q_OK && (n <= 0 || n % 128 != 0 || ldc < n)) rc = FP8Q_EINVAL;
  if (rc == FP8Q_OK) rc = check_proj(w_q, w_scale, out, n, ldc);
  if (rc != FP8Q_OK) return rc;
  if (k <= kPersistentMaxK) {
    ProjSet ps = {};
    ps.w[0] = w_q;
    ps.ws[0] = w_scale;
    ps.out[0] = out;
    ps.ldc[0] = ldc;
    ps.strip_end[0] = n / 16;
    ps.count = 1;
    const ActSrc act = {a_q, a_scale, nullptr, nullptr, nullptr};
    return run_persistent<false>(act, ps, m, k, stream);
  }
  return launch_gemm<4, 5>(a_q, a_scale, w_q, w_scale, out, m, n, k, ldc, stream);
}

extern "C" int w8a8_block_gemm_grouped(const uint8_t* a_q, const float* a_scale,
                                       const fp8q_gemm_proj* projs, int32_t count, int32_t m,
                                       int32_t k, hipStream_t stream) {
  if (count < 1 || count > kMaxProj) return FP8Q_EINVAL;
  if (!projs) return FP8Q_ENULL;
  int rc = check_gemm_common(a_q, a_scale, m, k);
  if (rc != FP8Q_OK) return rc;
  int64_t strips = 0;
  for (int p = 0; p < count; ++p) {
    rc = check_proj(projs[p].w_q, projs[p].w_scale, projs[p].out, projs[p].n, projs[p].ldc);
    if (rc != FP8Q_OK) return rc;
    strips += projs[p].n / 16;
  }
  if (strips > 0x7FFFFFFF) return FP8Q_EINVAL;
  if (k > kPersistentMaxK) {
    for (int p = 0; p < count; ++p) {
      rc = launch_gemm<4, 5>(a_q, a_scale, projs[p].w_q, projs[p].w_scale, projs[p].out, m,
                             projs[p].n, k, projs[p].ldc, stream);
      if (rc != FP8Q_OK) return rc;
    }
    return FP8Q_OK;
  }
  ProjSet ps = {};
  int end = 0;
  for (int p = 0; p < count; ++p) {
    ps.w[p] = projs[p].w_q;
    ps.ws[p] = projs[p].w_scale;
    ps.out[p] = projs[p].out;
    ps.ldc[p] = projs[p].ldc;
    end += projs[p].n / 16;
    ps.strip_end[p] = end;
  }
  ps.count = count;
  const ActSrc act = {a_q, a_scale, nullptr, nullptr, nullptr};
  return run_persistent<false>(act, ps, m, k, stream);
}

extern "C" int fp8_quant_w8a8_gemm_grouped(const uint16_t* a, uint8_t* a_q, float* a_scale,
                                           const fp8q_gemm_proj* projs, int32_t count,
                                           int32_t m, int32_t k, hipStream_t stream) {
  if (count < 1 || count > kMaxProj) return FP8Q_EINVAL;
  if (m < 1 || m > 16 || k <= 0 || k % 128 != 0 || k > kMaxGemmK) return FP8Q_EINVAL;
  if (!a || !projs) return FP8Q_ENULL;
  if ((a_q == nullptr) != (a_scale == nullptr)) return FP8Q_ENULL;
  // beyond the persistent kernel's K the quantizer and the GEMM run as two launches, through
  // the caller's code/scale buffers
  if (k > kPersistentMaxK && a_q == nullptr) return FP8Q_ENULL;
  if (!aligned(a, 16) || (a_q && (!aligned(a_q, 16) || !aligned(a_scale, 4))))
    return FP8Q_EALIGN;
  ProjSet ps = {};
  int64_t end = 0;
  for (int p = 0; p < count; ++p) {
    const int rc = check_proj(projs[p].w_q, projs[p].w_scale, projs[p].out, projs[p].n,
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
  if (k > kPersistentMaxK) {
    int rc = fp8_group_quant(a, a_q, a_scale, m, k, stream);
    if (rc == FP8Q_OK) rc = w8a8_block_gemm_grouped(a_q, a_scale, projs, count, m, k, stream);
    return rc;
  }
  const ActSrc act = {nullptr, nullptr, a, a_q, a_scale};
  return run_persistent<true>(act, ps, m, k, stream);
}
