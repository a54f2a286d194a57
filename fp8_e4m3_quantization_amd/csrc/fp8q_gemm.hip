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
// wave together with its row scales, so the LDS it needs does not grow with k).
// Rows >= m are fed zeros and never stored, so only (m-1)*ldc + n elements are written.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>
#include <utility>

#include "fp8q.h"
#include "fp8q_device.h"
#include "fp8q_gemm_common.h"
#include "fp8q_launch.h"

#pragma clang fp contract(off)

namespace fp8q {
namespace {

constexpr int kMaxGemmK = 131072;

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
  __shared__ float s_part[kWaves * 4 * 64];
  const int groups = k >> 7;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n0 = blockIdx.x * 16;

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
  // The 4 output rows this lane's accumulators hold: r0 .. r0 + 3.  Their activation scales
  // are read per group from the token-major grid (L2-resident: at most 16 * k/128 floats);
  // rows >= m read row m - 1 (in bounds) and are weighted by zero.
  const int r0 = 4 * (lane >> 4);
  const float* asr[4];
  float live[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    asr[j] = a_scale + int64_t(min(r0 + j, m - 1)) * groups;
    live[j] = r0 + j < m ? 1.0f : 0.0f;
  }

  const int g_begin = (groups * wv) / kWaves;
  const int g_end = (groups * (wv + 1)) / kWaves;
  v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
  const v8i zero8 = {0, 0, 0, 0, 0, 0, 0, 0};

  auto step = [&](const v8i& a, const v8i& b, float ws, const float4& as) {
    const v4f c = mfma_group(a, b);
    acc[0] = __builtin_fmaf(c[0], as.x * ws, acc[0]);
    acc[1] = __builtin_fmaf(c[1], as.y * ws, acc[1]);
    acc[2] = __builtin_fmaf(c[2], as.z * ws, acc[2]);
    acc[3] = __builtin_fmaf(c[3], as.w * ws, acc[3]);
  };
  auto row_scales = [&](int g) {
    return make_float4(asr[0][g] * live[0], asr[1][g] * live[1], asr[2][g] * live[2],
                       asr[3][g] * live[3]);
  };

  int g = g_begin;
  for (; g + kChunk <= g_end; g += kChunk) {
    v8i b[kChunk], a[kChunk];
    float4 as[kChunk];
#pragma unroll
    for (int u = 0; u < kChunk; ++u) b[u] = load32(wp + int64_t(g + u) * 128);
#pragma unroll
    for (int u = 0; u < kChunk; ++u) a[u] = a_live ? load32(ap + int64_t(g + u) * 128) : zero8;
#pragma unroll
    for (int u = 0; u < kChunk; ++u) as[u] = row_scales(g + u);
#pragma unroll
    for (int u = 0; u < kChunk; ++u) step(a[u], b[u], wsp[g + u], as[u]);
  }
  for (; g < g_end; ++g) {
    const v8i b = load32(wp + int64_t(g) * 128);
    const v8i a = a_live ? load32(ap + int64_t(g) * 128) : zero8;
    step(a, b, wsp[g], row_scales(g));
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
// Weight loads go through a buffer descriptor per strip (make_strip_rsrc), with the
// default cache policy.
constexpr int kGemmAux = 0;

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

// K split across workgroups (parts > 1; used when there are too few strips to give every
// CU a full share).  The grid is `parts` equal sets of workgroups; set p multiplies groups
// [G*p/parts, G*(p+1)/parts) of every strip it walks, its waves splitting that range, and
// writes the strip's part sum (the 16x16 fp32 tile in accumulator order) to
// partial[strip][p].  At the end of the kernel each workgroup counts its strips in; the one
// that completes a strip's count sums the parts in the order p = 0, 1, ... (the same sum
// whichever workgroup arrives last), writes bf16 and sets the count back to zero, so the
// counts are zero again for the next launch.  No workgroup ever waits for another.
struct SplitK {
  float* partial;   // [total_strips][parts][256]
  uint32_t* count;  // [total_strips]
  int parts;
};

template <int kGpw, int kDepth, int kAux, int kRound, bool kQuant, bool kSplit>
__global__ __launch_bounds__(64 * kPWaves) void w8a8_persistent_kernel(
    ActSrc act, ProjSet ps, int m, int k, int total_strips, int half_from, SplitK sk) {
  static_assert(kRound % (kDepth + 1) == 0, "buffer index must be static within a round");
  static_assert(kRound * 256 == kPWaves * 64 * 2, "reduce: two outputs per lane");
  static_assert(!(kQuant && kSplit), "the fused quantizer runs unsplit");
  __shared__ float s_part[2][kRound * kPWaves * 4 * 64];
  __shared__ uint4 s_tile[kPWaves * ActTile<kQuant ? 16 : 8>::kUints];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int groups = k >> 7;
  // this workgroup's set (K part) and its place in the set
  const int parts = kSplit ? sk.parts : 1;
  const int set_size = int(gridDim.x) / parts;
  const int kpart = kSplit ? int(blockIdx.x) / set_size : 0;
  const int in_set = kSplit ? int(blockIdx.x) % set_size : int(blockIdx.x);
  const int gb = (groups * kpart) / parts;
  const int gp = (groups * (kpart + 1)) / parts - gb;  // groups of this K part
  const int g0 = gb + (gp * wv) / kPWaves;
  const int cnt = gb + (gp * (wv + 1)) / kPWaves - g0;  // 0 <= cnt <= kGpw
  const int row = lane & 15, koff = (lane >> 4) * 32;
  int goff[kGpw];  // first k of slice group u (a short slice re-reads its last group,
                   // whose activation fragment below is zero)
#pragma unroll
  for (int u = 0; u < kGpw; ++u) goff[u] = (g0 + max(0, min(u, cnt - 1))) * 128;

  // work items: strips, the last round's halved (never in a K split, whose parts' tiles
  // are summed per strip)
  const int total_items = kSplit ? total_strips : item_count(total_strips, half_from);
  auto fetch = [&](int s, Slice<kGpw>& sl) {
    const bool valid = s < total_items;
    const StripItem it = strip_item(valid ? s : total_items - 1, kSplit ? total_strips : half_from);
    int p, n0;
    locate_strip(ps, it.strip, &p, &n0);
    const __amdgpu_buffer_rsrc_t r =
        make_strip_rsrc(ps.w[p] + int64_t(n0 + it.col0) * k, k, valid, it.cols);
    const_float* wsp = (const_float*)(ps.ws[p] + int64_t(n0 >> 7) * groups);
#pragma unroll
    for (int u = 0; u < kGpw; ++u) sl.b[u] = buffer_load32<kAux>(r, row * k + koff + goff[u]);
#pragma unroll
    for (int u = 0; u < kGpw; ++u) sl.ws[u] = wsp[goff[u] >> 7];
  };

  const int stride = set_size;
  const int first = first_strip(in_set, stride);
  const int nit = (total_items - first + stride - 1) / stride;
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
        const int strip = first + (i + j) * stride;
        if constexpr (kSplit) {
          // device-scope stores: written at the point where every XCD sees them
          float* dst = sk.partial + (int64_t(strip) * parts + kpart) * 256 + q0 * 64 + lane;
          __hip_atomic_store(dst, sum[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(dst + 64, sum[1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          const StripItem it = strip_item(strip, half_from);  // `strip` is an item here
          int p, n0;
          locate_strip(ps, it.strip, &p, &n0);
          uint16_t* o = ps.out[p] + n0 + it.col0 + (lane & 15);
          const int ldc = ps.ldc[p];
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            const int r = 4 * (lane >> 4) + q0 + x;
            if (r < m && (lane & 15) < it.cols) o[int64_t(r) * ldc] = f32_to_bf16_rne(sum[x]);
          }
        }
      }
    }
    par ^= 1;
  }

  if constexpr (kSplit) {
    // Count this workgroup's strips in, then finish every strip whose count it completed.
    // The part tiles and the counts are touched only by device-scope atomic accesses, which
    // are performed where every XCD sees them; each wave waits until its tile stores have
    // completed (acknowledged at that scope) before the barrier after which the counts are
    // raised, and a finishing workgroup reads the tiles only after its count returned.  A
    // device-scope fence would instead write back and invalidate the whole L2 of the XCD,
    // once per workgroup, which costs far more than the split saves.
    __shared__ int s_last[64 * kPWaves];
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int c0 = 0; c0 < nit; c0 += 64 * kPWaves) {
      const int t = c0 + int(threadIdx.x);
      if (t < nit) {
        const int strip = first + t * stride;
        const uint32_t before = __hip_atomic_fetch_add(sk.count + strip, 1u, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
        s_last[threadIdx.x] = before == uint32_t(parts - 1) ? strip : -1;
      }
      __syncthreads();
      const int nc = min(64 * kPWaves, nit - c0);
      for (int i = 0; i < nc; ++i) {
        const int strip = s_last[i];  // uniform
        if (strip < 0) continue;
        if (threadIdx.x < 256) {
          const float* src = sk.partial + int64_t(strip) * parts * 256 + threadIdx.x;
          float sum = 0.0f;
          for (int q = 0; q < parts; ++q)
            sum += __hip_atomic_load(src + q * 256, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const int l = threadIdx.x & 63;
          const int r = 4 * (l >> 4) + (threadIdx.x >> 6);
          int p, n0;
          locate_strip(ps, strip, &p, &n0);
          if (r < m) ps.out[p][int64_t(r) * ps.ldc[p] + n0 + (l & 15)] = f32_to_bf16_rne(sum);
        }
        if (threadIdx.x == 0)
          __hip_atomic_store(sk.count + strip, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------------
// Staged form (k a multiple of 1024, k <= 8192, K not split): the same strip walk and
// arithmetic, with the weight stream copied global -> LDS in pieces.  A piece is 1 KB (8
// K-groups) of each of an item's 16 weight rows; piece p of every item holds groups 8p ..
// 8p + 7, and wave w multiplies group 8p + w of it, so wave w keeps the activation
// fragments of groups w, w + 8, ... in registers.  The copies are the buffer unit's own
// (buffer_load ... lds), one instruction per weight row and piece: 1 KB of contiguous bytes,
// whole lines, non-temporal.  Straight into the MFMA operand layout each load instruction
// would instead touch 16 rows in half lines; measured as a plain read of the four decode
// projections' 178 MB on MI355X, that pattern runs at 5.4 TB/s and whole 1 KB rows at
// 6.0 TB/s, the rate of the best plain stream, which also needs few bytes in flight per CU
// (the one piece ahead here: 16 KB).  Lane i of a row's copy loads the row's 16-byte chunk
// i ^ r (r = row), so chunk c of row r lands at position c ^ r and the fragment reads (one
// chunk of 16 rows per 16 lanes) are free of bank conflicts.  The copies rotate through
// four 16 KB slots, one piece ahead, with one barrier per piece: the barrier of piece q
// follows each wave's wait for its own copies of piece q, and the slot piece q + 1 is copied
// into was last read for piece q - 3, which every wave finished before the barrier of
// piece q - 2.  The waits are explicit vmcnt counts, so every vector memory instruction
// between a copy and its wait is issued unconditionally: the round's bf16 stores are
// buffer stores whose dropped lanes take an offset past the descriptor.
constexpr int kStageSlot = 16 * 1024;
constexpr uint32_t kDropOffset = 0xFFFFFFF0u;  // past every descriptor: the store is dropped
constexpr int kNonTemporal = 2;                // cache-policy bits of the copies: nt
typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt vmcnt(kN) lgkmcnt(0) (expcnt untouched), then s_barrier; nothing is moved across.
template <int kN>
__device__ __forceinline__ void wait_copies_then_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((kN & 15) | (7 << 4) | ((kN >> 4) << 14));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Calls f(std::integral_constant<int, i>()) for i = 0 .. kN - 1 (a loop whose index is a
// compile-time constant in the body).
template <int kN, typename Fn, int... kI>
__device__ __forceinline__ void static_for_impl(Fn&& f, std::integer_sequence<int, kI...>) {
  (f(std::integral_constant<int, kI>()), ...);
}
template <int kN, typename Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
  static_for_impl<kN>(f, std::make_integer_sequence<int, kN>());
}

// The activation a staged launch multiplies: E4M3 codes with their row scales, bf16 that the
// launch quantizes itself (the fused form), or bf16 taken as is (the W8A16 tier).
enum StagedAct { kActCodes = 0, kActQuantize = 1, kActBf16 = 2 };

template <int kGpw, int kAct, int kDepth>
__device__ __forceinline__ void staged_body(const ActSrc& act, const ProjSet& ps, int m, int k,
                                            int total_strips, int half_from) {
  static_assert(kDepth >= 1 && kDepth <= 3, "copies at most three pieces ahead of four slots");
  constexpr bool kQuant = kAct == kActQuantize;
  constexpr int kRound = 4;
  constexpr int kPartFloats = kRound * kPWaves * 4 * 64;
  using Tile = ActTile<kAct == kActCodes ? 8 : 16>;
  static_assert(kRound * 256 == kPWaves * 64 * 2, "reduce: two outputs per lane");
  // four slots as four arrays: every slot index below is a compile-time constant, so a
  // fragment read is seen not to touch the slot whose copies are still in flight
  __shared__ __attribute__((aligned(16))) uint8_t s_slot0[kStageSlot];
  __shared__ __attribute__((aligned(16))) uint8_t s_slot1[kStageSlot];
  __shared__ __attribute__((aligned(16))) uint8_t s_slot2[kStageSlot];
  __shared__ __attribute__((aligned(16))) uint8_t s_slot3[kStageSlot];
  auto slot_at = [&](int t) -> uint8_t* {
    switch (t & 3) {
      case 0: return s_slot0;
      case 1: return s_slot1;
      case 2: return s_slot2;
      default: return s_slot3;
    }
  };
  // the partial tiles of a round, and the waves' activation tiles.  Every LDS array is
  // addressed from its own name (no pointer chosen at run time), so the compiler sees which
  // arrays the copies in flight cannot touch and does not wait for them before reading
  // these.
  __shared__ __attribute__((aligned(16))) float s_part[kPartFloats];
  __shared__ uint4 s_tile[kPWaves * Tile::kUints];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int groups = k >> 7;
  const int row = lane & 15, koff = (lane >> 4) * 32;
  const int r0 = 4 * (lane >> 4);

  const int total_items = item_count(total_strips, half_from);
  const int stride = int(gridDim.x);
  const int first = first_strip(int(blockIdx.x), stride);
  const int nit = (total_items - first + stride - 1) / stride;
  if (nit <= 0) return;

  // Copies of piece p of this workgroup's item i (i >= nit: a zero-size buffer, zeros
  // written to the slot and no memory touched) into slot t % 4, t = i kGpw + p (items are
  // walked in rounds of 4 from a multiple of 4, so t % 4 is known at compile time from the
  // item's place in the round); returns the weight block scale of the group this wave
  // multiplies in that piece.
  auto issue = [&](int i, int p, int t) {
    const bool valid = i < nit;
    const StripItem it = strip_item(first + (valid ? i : 0) * stride, half_from);
    int pj, n0;
    locate_strip(ps, it.strip, &pj, &n0);
    const __amdgpu_buffer_rsrc_t r =
        make_strip_rsrc(ps.w[pj] + int64_t(n0 + it.col0) * k, k, valid, it.cols);
    uint8_t* slot = slot_at(t);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int wr = 2 * wv + h;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(slot + wr * 1024), 16,
                                               wr * k + p * 1024 + 16 * (lane ^ wr), 0, 0,
                                               kNonTemporal);
    }
    const_float* wsp = (const_float*)(ps.ws[pj] + int64_t(n0 >> 7) * groups);
    return wsp[8 * p + wv];
  };


  // Reduce of the round whose partial tiles are in `part` (round items i0 ..): wave w sums
  // half of round item w / 2 (2 outputs per lane) over the waves in order and stores them as
  // bf16.  Both store instructions are issued whatever the item (with `live` false, or past
  // the last item, every lane stores past the descriptor and is dropped), so the count of
  // vector memory instructions between a copy and its wait never depends on the data.
  auto reduce_sum = [&](const float* part, float (&sum)[2]) {
    const int j = wv >> 1, q0 = (wv & 1) * 2;  // wave-uniform
    sum[0] = sum[1] = 0.0f;
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int w = 0; w < kPWaves; ++w) sum[x] += part[((j * kPWaves + w) * 4 + q0 + x) * 64 + lane];
  };
  auto reduce_store = [&](const float (&sum)[2], int i0, bool live) {
    const int j = wv >> 1, q0 = (wv & 1) * 2;  // wave-uniform
    const bool live_item = live && i0 + j < nit;
    const StripItem it = strip_item(first + (live_item ? i0 + j : 0) * stride, half_from);
    int pj, n0;
    locate_strip(ps, it.strip, &pj, &n0);
    const __amdgpu_buffer_rsrc_t o =
        __builtin_amdgcn_make_buffer_rsrc(ps.out[pj], 0, 0x7FFFFFFF, kBufferDword3);
    const int ldc = ps.ldc[pj];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int r = 4 * (lane >> 4) + q0 + x;
      const bool st = live_item && r < m && (lane & 15) < it.cols;
      const uint32_t off = st ? uint32_t(r * ldc + n0 + it.col0 + (lane & 15)) * 2u : kDropOffset;
      __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(sum[x]), o, off, 0, 0);
    }
  };

  // Activation: the raw loads of every group go out first, the first pieces' copies right
  // behind them; then the fragments of every group, through the wave's LDS tile (as in the
  // persistent form).
  uint4* tile = s_tile + wv * Tile::kUints;
  const v8i zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
  v8i a[kGpw];
  float4 as[kGpw];
  float scv[kGpw];  // kQuant: this lane's row scale of each group
  uint4 af[kGpw][4];  // kActBf16: this lane's 32 bf16 of each group
  v4u raw[kGpw][Tile::kLoads];
  float4 rs[kGpw];  // kActCodes: the row scales of lanes' four output rows
  // Every group's raw loads up front, except in the fused form with more than six groups per
  // wave (K > 6144), where all the bf16 tiles and the codes would not fit in registers: there
  // each group is loaded and quantized in turn after the copies (the fused form still spills
  // from six groups per wave on, 96-328 bytes a lane).
  constexpr bool kAllLoadsFirst = !(kQuant && kGpw > 6);
  auto load_group = [&](int u) {
    const int goff = (8 * u + wv) * 128;  // first k of group 8u + wv
    if constexpr (kAct != kActCodes) {
      Tile::load(reinterpret_cast<const uint8_t*>(act.a_bf16) + 2 * goff, 2 * int64_t(k), m,
                 lane, raw[u]);
    } else {
      Tile::load(act.a_q + goff, k, m, lane, raw[u]);
      const int g = goff >> 7;
      rs[u].x = act.a_scale[int64_t(min(r0 + 0, m - 1)) * groups + g];
      rs[u].y = act.a_scale[int64_t(min(r0 + 1, m - 1)) * groups + g];
      rs[u].z = act.a_scale[int64_t(min(r0 + 2, m - 1)) * groups + g];
      rs[u].w = act.a_scale[int64_t(min(r0 + 3, m - 1)) * groups + g];
    }
  };
  if constexpr (kAllLoadsFirst) {
#pragma unroll
    for (int u = 0; u < kGpw; ++u) load_group(u);
  }
  // The first kDepth + 1 pieces (every slot with three ahead) are copied before the
  // activation fragments are made: the fused form's quantization alone is about 6 VALU
  // operations per element, 160 elements per lane, microseconds during which these copies
  // are the only bytes in flight.  The first item's first piece then issues no copy (its
  // piece kDepth is already out).
  float wsq[4];  // weight block scales of the pieces in flight, by slot
  static_for<kDepth + 1>([&](auto dc) {
    constexpr int d = decltype(dc)::value;
    wsq[d & 3] = issue(d / kGpw, d % kGpw, d);
  });
  __builtin_amdgcn_sched_barrier(0);  // keep the copies ahead of the activation math

  auto make_fragments = [&](int u) {
    if constexpr (kAct == kActBf16) {
      // rows >= m repeat row m - 1 (Tile::load): finite, computed and never stored
      Tile::exchange(tile, raw[u], lane, koff >> 3, af[u]);
    } else if constexpr (kAct == kActCodes) {
      uint4 f[2];
      Tile::exchange(tile, raw[u], lane, koff >> 4, f);
      const v8i fr = {int(f[0].x), int(f[0].y), int(f[0].z), int(f[0].w),
                      int(f[1].x), int(f[1].y), int(f[1].z), int(f[1].w)};
      a[u] = row < m ? fr : zero8;
      as[u].x = r0 + 0 < m ? rs[u].x : 0.0f;
      as[u].y = r0 + 1 < m ? rs[u].y : 0.0f;
      as[u].z = r0 + 2 < m ? rs[u].z : 0.0f;
      as[u].w = r0 + 3 < m ? rs[u].w : 0.0f;
    } else {
      uint4 x[4];
      Tile::exchange(tile, raw[u], lane, koff >> 3, x);
      float amax = fmaxf(fmaxf(absmax8(x[0]), absmax8(x[1])), fmaxf(absmax8(x[2]), absmax8(x[3])));
      amax = fmaxf(amax, __shfl_xor(amax, 16));
      amax = fmaxf(amax, __shfl_xor(amax, 32));
      const float sc = group_scale_from_amax(amax);
      const float y = 1.0f / sc;  // IEEE division: RN(1/s)
      const uint2 c0 = quant8<true>(x[0], sc, y), c1 = quant8<true>(x[1], sc, y);
      const uint2 c2 = quant8<true>(x[2], sc, y), c3 = quant8<true>(x[3], sc, y);
      v8i f;
      f[0] = int(c0.x); f[1] = int(c0.y); f[2] = int(c1.x); f[3] = int(c1.y);
      f[4] = int(c2.x); f[5] = int(c2.y); f[6] = int(c3.x); f[7] = int(c3.y);
      a[u] = row < m ? f : zero8;
      // row r's scale sits in lane r (and r+16, r+32, r+48)
      const float s0 = __shfl(sc, r0 + 0), s1 = __shfl(sc, r0 + 1);
      const float s2 = __shfl(sc, r0 + 2), s3 = __shfl(sc, r0 + 3);
      as[u].x = r0 + 0 < m ? s0 : 0.0f;
      as[u].y = r0 + 1 < m ? s1 : 0.0f;
      as[u].z = r0 + 2 < m ? s2 : 0.0f;
      as[u].w = r0 + 3 < m ? s3 : 0.0f;
      scv[u] = sc;
    }
  };

#pragma unroll
  for (int u = 0; u < kGpw; ++u) {
    if constexpr (!kAllLoadsFirst) load_group(u);
    make_fragments(u);
  }

  // Piece p of round item j (t = j kGpw + p), round items from i.  With one piece ahead the
  // next copies are issued before this piece's wait (one piece stays in flight while
  // waiting); with more, after the barrier, when every wave has finished reading the slot
  // they go to (piece t + kDepth - 4 <= t - 1).  The wait: newer than this piece's copies
  // are the copies of the next kDepth - 1 pieces (kDepth with one piece ahead), and for
  // pieces 1 .. kDepth of a round the two stores of the previous round's reduce (issued in
  // piece 0 after the copies of piece kDepth).
  auto piece = [&](auto jc, auto pc, int i, v4f& acc, auto first_item) {
    constexpr int j = decltype(jc)::value, p = decltype(pc)::value, t = j * kGpw + p;
    auto issue_ahead = [&]() {
      if constexpr (!(decltype(first_item)::value && t == 0))
        wsq[(t + kDepth) & 3] = issue(i + j + (p + kDepth) / kGpw, (p + kDepth) % kGpw, t + kDepth);
    };
    if constexpr (kDepth == 1) issue_ahead();
    constexpr int kAhead = kDepth == 1 ? 2 : 2 * (kDepth - 1);
    if constexpr (t >= 1 && t <= kDepth)
      wait_copies_then_barrier<kAhead + 2>();
    else
      wait_copies_then_barrier<kAhead>();
    // (round start: the previous round's partial tiles are read before the copies are
    // issued, which the compiler would otherwise make wait for them)
    float sum[2];
    if constexpr (t == 0) reduce_sum(s_part, sum);
    if constexpr (kDepth > 1) issue_ahead();
    if constexpr (t == 0) reduce_store(sum, i - kRound, i > 0);
    const uint8_t* slot = slot_at(t) + row * 1024;
    const int c0 = 8 * wv + 2 * (lane >> 4);
    const v4u x = *reinterpret_cast<const v4u*>(slot + 16 * (c0 ^ row));
    const v4u y = *reinterpret_cast<const v4u*>(slot + 16 * ((c0 + 1) ^ row));
    const v8i b = {int(x[0]), int(x[1]), int(x[2]), int(x[3]),
                   int(y[0]), int(y[1]), int(y[2]), int(y[3])};
    const float wsc = wsq[t & 3];
    if constexpr (kAct == kActBf16) {
      // the W8A16 tier: the 32 codes widened to bf16 (exact), four bf16 MFMAs over the group,
      // its partial times the block scale (the activation carries no scale)
      v4f c = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int q = 0; q < 4; ++q)
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf16, af[p][q]),
                                                    widen8(uint32_t(b[2 * q]), uint32_t(b[2 * q + 1])),
                                                    c, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = __builtin_fmaf(c[q], wsc, acc[q]);
    } else {
      const v4f c = mfma_group(a[p], b);
      acc[0] = __builtin_fmaf(c[0], as[p].x * wsc, acc[0]);
      acc[1] = __builtin_fmaf(c[1], as[p].y * wsc, acc[1]);
      acc[2] = __builtin_fmaf(c[2], as[p].z * wsc, acc[2]);
      acc[3] = __builtin_fmaf(c[3], as[p].w * wsc, acc[3]);
    }
  };
  // One partial buffer: a round's reduce reads it in the next round's first piece, after that
  // piece's barrier, and the next partial tile goes in at the end of the round's first item,
  // after the barriers of its later pieces (with one piece per item, after one more barrier).
  auto item = [&](auto jc, int i, auto first_item) {
    constexpr int j = decltype(jc)::value;
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
    static_for<kGpw>([&](auto pc) { piece(jc, pc, i, acc, first_item); });
    if constexpr (kGpw == 1 && j == 0) lds_barrier();
#pragma unroll
    for (int q = 0; q < 4; ++q) s_part[((j * kPWaves + wv) * 4 + q) * 64 + lane] = acc[q];
  };

  // The first item on its own (its first piece issues no copy), then the rest.  In the
  // first round the wait counts over-wait for at most the first kDepth pieces.
  item(std::integral_constant<int, 0>(), 0, std::true_type());
  for (int i = 0; i < nit; i += kRound)
    static_for<kRound>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      if (i + j < nit && (j > 0 || i > 0)) item(jc, i, std::false_type());  // uniform
    });
  // the last round's reduce, then (fused, optional) the codes and scales
  lds_barrier();
  {
    float sum[2];
    reduce_sum(s_part, sum);
    reduce_store(sum, ((nit - 1) / kRound) * kRound, true);
  }
  if constexpr (kQuant) {
    if (act.q_out != nullptr) {
#pragma unroll
      for (int u = 0; u < kGpw; ++u) {
        const int g = 8 * u + wv;
        if (row < m && (row * groups + g) % stride == int(blockIdx.x)) {
          uint4* qo = reinterpret_cast<uint4*>(act.q_out + int64_t(row) * k + g * 128 + koff);
          qo[0] = make_uint4(uint32_t(a[u][0]), uint32_t(a[u][1]), uint32_t(a[u][2]), uint32_t(a[u][3]));
          qo[1] = make_uint4(uint32_t(a[u][4]), uint32_t(a[u][5]), uint32_t(a[u][6]), uint32_t(a[u][7]));
          if (lane < 16) act.s_out[int64_t(row) * groups + g] = scv[u];
        }
      }
    }
  }
  // no copy into LDS may be in flight when the workgroup ends (the last issued pieces)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int kGpw, bool kQuant, int kDepth>
__global__ __launch_bounds__(64 * kPWaves) void w8a8_staged_kernel(ActSrc act, ProjSet ps, int m,
                                                                    int k, int total_strips,
                                                                    int half_from) {
  staged_body<kGpw, kQuant ? kActQuantize : kActCodes, kDepth>(act, ps, m, k, total_strips,
                                                                half_from);
}

// The W8A16 tier (1..4 bf16 activation rows) in the same staged form.
template <int kGpw, int kDepth>
__global__ __launch_bounds__(64 * kPWaves) void w8a16_staged_kernel(ActSrc act, ProjSet ps, int m,
                                                                     int k, int total_strips,
                                                                     int half_from) {
  staged_body<kGpw, kActBf16, kDepth>(act, ps, m, k, total_strips, half_from);
}

template <int kWaves, int kChunk>
int launch_gemm(const uint8_t* a_q, const float* a_scale, const uint8_t* w_q,
                const float* w_scale, uint16_t* out, int m, int n, int k, int ldc,
                hipStream_t stream) {
  launch((w8a8_gemm_kernel<kWaves, kChunk>), dim3(n / 16), dim3(64 * kWaves), 0, stream, a_q,
         a_scale, w_q, w_scale, out, m, k, ldc);
  return launch_status();
}

template <int kGpw, bool kQuant, bool kSplit>
int launch_persistent(const ActSrc& act, const ProjSet& ps, int m, int k, int total,
                      const SplitK& sk, int grid, hipStream_t stream) {
  // a short slice per wave (split K) keeps more strips in flight to cover the latency
  constexpr int kDepth = (kSplit && kGpw <= 2) ? 3 : 1;
  constexpr int kRound = 4;
  const int half_from = kSplit ? total : halved_from(total, grid);
  launch((w8a8_persistent_kernel<kGpw, kDepth, kGemmAux, kRound, kQuant, kSplit>),
         dim3(grid), dim3(64 * kPWaves), 0, stream, act, ps, m, k, total, half_from, sk);
  return launch_status();
}

#ifndef FP8Q_STAGE_DEPTH
#define FP8Q_STAGE_DEPTH 3
#endif
template <int kGpw, bool kQuant>
int launch_staged(const ActSrc& act, const ProjSet& ps, int m, int k, int total, int grid,
                  hipStream_t stream) {
  launch((w8a8_staged_kernel<kGpw, kQuant, FP8Q_STAGE_DEPTH>), dim3(grid), dim3(64 * kPWaves), 0,
         stream, act, ps, m, k, total, halved_from(total, grid));
  return launch_status();
}

template <int kGpw>
int launch_w8a16_staged(const uint16_t* a, const ProjSet& ps, int m, int k, int total, int grid,
                        hipStream_t stream) {
  const ActSrc act = {nullptr, nullptr, a, nullptr, nullptr};
  launch((w8a16_staged_kernel<kGpw, FP8Q_STAGE_DEPTH>), dim3(grid), dim3(64 * kPWaves), 0, stream,
         act, ps, m, k, total, halved_from(total, grid));
  return launch_status();
}

// Persistent kernel for k <= 8 * 8 * 128 (each wave holds at most 8 groups).  kSplit:
// sk.parts > 1 sets of workgroups split K (the grid is parts * set size).  Unsplit with k a
// multiple of 1024 it runs in the staged form.
template <bool kQuant, bool kSplit = false>
int run_persistent(const ActSrc& act, const ProjSet& ps, int m, int k, hipStream_t stream,
                   const SplitK& sk = SplitK{nullptr, nullptr, 1}) {
  const int total = ps.strip_end[ps.count - 1];
  if (!kSplit && k % 1024 == 0) {
    const int grid = total < num_cus() ? total : num_cus();
    switch (k / 1024) {
      case 1: return launch_staged<1, kQuant>(act, ps, m, k, total, grid, stream);
      case 2: return launch_staged<2, kQuant>(act, ps, m, k, total, grid, stream);
      case 3: return launch_staged<3, kQuant>(act, ps, m, k, total, grid, stream);
      case 4: return launch_staged<4, kQuant>(act, ps, m, k, total, grid, stream);
      case 5: return launch_staged<5, kQuant>(act, ps, m, k, total, grid, stream);
      case 6: return launch_staged<6, kQuant>(act, ps, m, k, total, grid, stream);
      case 7: return launch_staged<7, kQuant>(act, ps, m, k, total, grid, stream);
      case 8: return launch_staged<8, kQuant>(act, ps, m, k, total, grid, stream);
      default: return FP8Q_EINVAL;
    }
  }
  const int parts = kSplit ? sk.parts : 1;
  const int part_groups = (k / 128 + parts - 1) / parts;
  const int gpw = (part_groups + kPWaves - 1) / kPWaves;
  const int set = total < num_cus() / parts ? total : num_cus() / parts;
  const int grid = set * parts;
  switch (gpw) {
    case 1: return launch_persistent<1, kQuant, kSplit>(act, ps, m, k, total, sk, grid, stream);
    case 2: return launch_persistent<2, kQuant, kSplit>(act, ps, m, k, total, sk, grid, stream);
    case 3: return launch_persistent<3, kQuant, kSplit>(act, ps, m, k, total, sk, grid, stream);
    case 4: return launch_persistent<4, kQuant, kSplit>(act, ps, m, k, total, sk, grid, stream);
    case 5: return launch_persistent<5, kQuant, kSplit>(act, ps, m, k, total, sk, grid, stream);
    case 6: return launch_persistent<6, kQuant, kSplit>(act, ps, m, k, total, sk, grid, stream);
    case 7: return launch_persistent<7, kQuant, kSplit>(act, ps, m, k, total, sk, grid, stream);
    case 8: return launch_persistent<8, kQuant, kSplit>(act, ps, m, k, total, sk, grid, stream);
    default: return FP8Q_EINVAL;
  }
}

constexpr int kPersistentMaxK = kPWaves * 8 * 128;

// K parts for `strips` 16-column strips of `groups` K-groups on `cus` CUs.  A launch
// costs a fixed part (about 7 us on MI355X at K = 5120, half of it the launch itself) plus
// about 1 us per round of strips; splitting K into two parts halves the groups each wave
// streams per strip and adds a partial-tile write, count and read.  Measured over N = 128 ..
// 8192 and 2..8 parts (K = 5120, 16 rows): two parts win (by 0.3 to 1.9 us) exactly when
// both parts' workgroups still run in one round, i.e. 2 * strips <= CUs, and more parts
// never beat two by more than noise; once a split adds a round it loses.  A part also needs
// a group per wave to stream (groups >= 16).
constexpr int kMaxParts = 2;

int split_parts(int strips, int groups, int cus) {
  return (2 * strips <= cus && groups >= 2 * kPWaves) ? kMaxParts : 1;
}

// Workspace of a split launch: the counts first (256-byte aligned), then the tiles.
uint64_t split_counts_bytes(int strips) { return (uint64_t(strips) * 4 + 255) & ~uint64_t(255); }
uint64_t split_workspace_bytes(int strips, int parts) {
  return parts <= 1 ? 0 : split_counts_bytes(strips) + uint64_t(strips) * parts * 256 * 4;
}

}  // namespace

int run_w8a16_staged(const uint16_t* a, const ProjSet& ps, int m, int k, hipStream_t stream) {
  const int total = ps.strip_end[ps.count - 1];
  const int grid = total < num_cus() ? total : num_cus();
  switch (k / 1024) {
    case 1: return launch_w8a16_staged<1>(a, ps, m, k, total, grid, stream);
    case 2: return launch_w8a16_staged<2>(a, ps, m, k, total, grid, stream);
    case 3: return launch_w8a16_staged<3>(a, ps, m, k, total, grid, stream);
    case 4: return launch_w8a16_staged<4>(a, ps, m, k, total, grid, stream);
    case 5: return launch_w8a16_staged<5>(a, ps, m, k, total, grid, stream);
    case 6: return launch_w8a16_staged<6>(a, ps, m, k, total, grid, stream);
    case 7: return launch_w8a16_staged<7>(a, ps, m, k, total, grid, stream);
    case 8: return launch_w8a16_staged<8>(a, ps, m, k, total, grid, stream);
    default: return FP8Q_EINVAL;
  }
}

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

namespace {
// The K split w8a8_block_gemm_ws uses for this shape on the current device (1: none).  K a
// multiple of 1024 runs unsplit in the staged form, which is faster there than the split
// persistent form (N = 1024, K = 5120, M = 16: 6.2 against 7.2 us).
int ws_parts(int32_t n, int32_t k) {
  if (k > kPersistentMaxK || k % 1024 == 0) return 1;
  return split_parts(n / 16, k / 128, num_cus());
}

// One projection with K split in `parts`: counts [n/16] (zero on entry, zero again on
// exit) and part tiles [n/16][parts][256] fp32.
int run_split(const uint8_t* a_q, const float* a_scale, const uint8_t* w_q,
              const float* w_scale, uint16_t* out, int32_t m, int32_t n, int32_t k,
              int32_t ldc, uint32_t* counts, float* tiles, int parts, hipStream_t stream) {
  ProjSet ps = {};
  ps.w[0] = w_q;
  ps.ws[0] = w_scale;
  ps.out[0] = out;
  ps.ldc[0] = ldc;
  ps.strip_end[0] = n / 16;
  ps.count = 1;
  const ActSrc act = {a_q, a_scale, nullptr, nullptr, nullptr};
  const SplitK sk = {tiles, counts, parts};
  return run_persistent<false, true>(act, ps, m, k, stream, sk);
}

// ---------------------------------------------------------- allocation-free K split
// w8a8_block_gemm_noalloc keeps the split's counts and part tiles in `scratch`, a static
// array of every device the library runs on (each device holds its own copy at its own
// address).  Host code never uses the array's name as an address: the device address is
// looked up once per device with hipGetSymbolAddress and kept in scratch_ptr.
constexpr uint64_t kScratchCountBytes = 4096;        // counts of up to 1024 strips
constexpr uint64_t kScratchTileBytes = 1u << 20;     // up to 1024 strips x parts of 1 KB
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) uint8_t scratch[kScratchCountBytes + kScratchTileBytes];

namespace {

std::mutex scratch_mu;
uint8_t* scratch_ptr[kMaxDevices] = {};

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, int n) {
  for (int i = int(blockIdx.x) * 256 + int(threadIdx.x); i < n; i += int(gridDim.x) * 256)
    p[i] = 0u;
}

// The current device's scratch address.  The first call on a device looks it up and
// enqueues a fill that zeroes the counts on `stream` (a kernel, so that a captured graph
// holds no memset node; the array also starts zeroed when the code object is loaded).
int scratch_on_device(hipStream_t stream, uint8_t** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FP8Q_EHIP;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FP8Q_EHIP;
    const LaunchEvents timed = g_next_launch_events;  // the fill is not the timed kernel
    g_next_launch_events = LaunchEvents();
    launch(zero_words_kernel, dim3(4), dim3(256), 0, stream, static_cast<uint32_t*>(p),
           int(kScratchCountBytes / 4));
    g_next_launch_events = timed;
    if (launch_status() != FP8Q_OK) return FP8Q_ELAUNCH;
    scratch_ptr[dev] = static_cast<uint8_t*>(p);
  }
  *out = scratch_ptr[dev];
  return FP8Q_OK;
}
}  // namespace

extern "C" int w8a8_block_gemm_workspace_size(int32_t m, int32_t n, int32_t k,
                                              uint64_t* bytes) {
  if (!bytes) return FP8Q_ENULL;
  *bytes = 0;
  if (m < 1 || m > 16 || k <= 0 || k % 128 != 0 || k > kMaxGemmK || n <= 0 || n % 128 != 0)
    return FP8Q_EINVAL;
  *bytes = split_workspace_bytes(n / 16, ws_parts(n, k));
  return FP8Q_OK;
}

extern "C" int w8a8_block_gemm_ws(const uint8_t* a_q, const float* a_scale,
                                  const uint8_t* w_q, const float* w_scale, uint16_t* out,
                                  int32_t m, int32_t n, int32_t k, int32_t ldc,
                                  void* workspace, uint64_t workspace_bytes,
                                  hipStream_t stream) {
  int rc = check_gemm_common(a_q, a_scale, m, k);
  if (rc == FP8Q_OK) rc = check_proj(w_q, w_scale, out, n, ldc);
  if (rc != FP8Q_OK) return rc;
  const int parts = ws_parts(n, k);
  if (parts <= 1) return w8a8_block_gemm(a_q, a_scale, w_q, w_scale, out, m, n, k, ldc, stream);
  if (!workspace) return FP8Q_ENULL;
  if (workspace_bytes < split_workspace_bytes(n / 16, parts)) return FP8Q_EINVAL;
  if (!aligned(workspace, 256)) return FP8Q_EALIGN;
  uint8_t* base = static_cast<uint8_t*>(workspace);
  return run_split(a_q, a_scale, w_q, w_scale, out, m, n, k, ldc,
                   reinterpret_cast<uint32_t*>(base),
                   reinterpret_cast<float*>(base + split_counts_bytes(n / 16)), parts, stream);
}

extern "C" int w8a8_block_gemm_noalloc(const uint8_t* a_q, const float* a_scale,
                                       const uint8_t* w_q, const float* w_scale, uint16_t* out,
                                       int32_t m, int32_t n, int32_t k, int32_t ldc,
                                       hipStream_t stream) {
  int rc = check_gemm_common(a_q, a_scale, m, k);
  if (rc == FP8Q_OK) rc = check_proj(w_q, w_scale, out, n, ldc);
  if (rc != FP8Q_OK) return rc;
  const int parts = ws_parts(n, k);
  if (parts <= 1) return w8a8_block_gemm(a_q, a_scale, w_q, w_scale, out, m, n, k, ldc, stream);
  const uint64_t strips = uint64_t(n / 16);
  if (strips * 4 > kScratchCountBytes || strips * uint64_t(parts) * 1024 > kScratchTileBytes)
    return FP8Q_EINVAL;
  uint8_t* base = nullptr;
  rc = scratch_on_device(stream, &base);
  if (rc != FP8Q_OK) return rc;
  return run_split(a_q, a_scale, w_q, w_scale, out, m, n, k, ldc,
                   reinterpret_cast<uint32_t*>(base),
                   reinterpret_cast<float*>(base + kScratchCountBytes), parts, stream);
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
