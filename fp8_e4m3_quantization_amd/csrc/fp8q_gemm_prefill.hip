// fp8q_gemm_prefill.hip -- block-scaled W8A8 GEMM for prefill widths (hundreds to thousands
// of activation rows): the dense, MFMA-bound form of the same arithmetic as the decode GEMM.
//
// fp8_residency.rs page, DenseFp8Inputs::w8a8_kernels (the W8A8 prefill arm is the
// per-token group quantizer followed by a block-scaled FP8 GEMM); fp8_act_quant.rs page,
// module doc (a 4593-token prefill); dispatch_proj_decode.rs page, module doc NUMERICS
// (E4M3 activations with per-token 1x128 FP32 scales times E4M3 weights with 128x128 FP32
// block scales, FP32 epilogue).
//
// Both kernels walk K one 128-wide group at a time; one v_mfma_f32_16x16x128_f8f6f4 covers
// one group of a 16 x 16 output tile, so every instruction's result is one group's partial
// and takes its scale a_scale[row, g] * w_scale[col/128, g] in one FMA per element.  The
// operand tiles of each group are copied global -> LDS by the buffer unit itself
// (buffer_load ... lds: no staging registers, no LDS store instructions) into one of two
// stages, the next group's copies landing while the current group multiplies.
//
// tile256 (the large shapes): one 512-thread workgroup per CU owns a 256 x 256 output tile,
// wave (wm, wn) of the 4 x 2 grid 64 x 128 of it (4 x 8 MFMA tiles).  A 256 x 256 tile
// copies half the operand bytes per flop of a 128 x 128 one, which the copy path (the
// texture/address unit, about 70 % busy with 128 x 128 tiles) needs, and 64 x 128 per wave
// reads 0.75 KB of LDS per MFMA.  The column loop is software-pipelined: column c + 1's
// weight fragment is read and column c - 1's products are scaled while column c
// multiplies, one group of four FMAs between MFMAs; after each group's barrier only B_0
// and the first two activation fragments are read before the first MFMA, each later
// fragment an MFMA ahead of its use.
// Both scales come from LDS (the weight block scale rides in the activation-scale copy),
// so no scalar load shares the LDS reads' wait counter.  When the tile count leaves the last
// round of workgroups at most half full, each of those last tiles is split into two
// 256 x 128 halves (wave tiles 64 x 64): twice as many work items, each half as long.
//
// tile128 (fewer than half a round of 256 x 256 tiles, e.g. a 1024-column projection):
// 256-thread workgroups, two per CU, each a 128 x 128 tile (2 x 2 waves of 64 x 64).
//
// Workgroups are ordered so that concurrently running ones share operand tiles:
// consecutive row tiles per column tile, and each XCD (workgroup ids are dealt to the 8
// XCDs round-robin) takes a contiguous stretch of that order for its own L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8q.h"
#include "fp8q_gemm_common.h"
#include "fp8q_launch.h"
#include "fp8q_math.h"

#pragma clang fp contract(off)

namespace fp8q {
namespace {

constexpr int kXcds = 8;

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// E4M3 x E4M3 -> FP32 over one 128-wide K-group of a 16 x 16 tile (no scaling).
__device__ __forceinline__ v4f mfma_group(v8i a, v8i b) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// Buffer descriptor over the rows [r0, min(rows, r0 + tile_rows)) of a [rows, k] byte
// matrix: reads past them return zeros without touching memory.  Its size is at most
// tile_rows * k bytes, which the host keeps below 2^31.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* base, int r0, int rows,
                                                            int k, int tile_rows) {
  const int valid = min(rows - r0, tile_rows);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base + int64_t(r0) * k), 0,
                                           valid > 0 ? valid * k : 0, kBufferDword3);
}

namespace tile256 {

constexpr int kBM = 256, kBN = 256, kThreads = 512;
constexpr int kCPitch = kBN + 8;          // bf16 elements per staged output row
constexpr int kSlab = 64 * kCPitch * 2;   // 64 staged output rows (bytes)
static_assert(kSlab >= kBM * 128, "a stage array holds one operand tile of one group");
constexpr int kGroupM = 4;                // row tiles per column tile in the walk order

// Two LDS stages.  The operand arrays are padded to kSlab so that the four of them also
// hold the four 64-row slabs of the staged bf16 output tile.  They are separate objects:
// the compiler can then see that a stage's operand reads never alias the copies landing
// in the other stage, and keeps those copies in flight.
struct Stages {
  uint8_t (&a0)[kSlab];
  uint8_t (&a1)[kSlab];
  uint8_t (&b0)[kSlab];
  uint8_t (&b1)[kSlab];
  float (&s0)[kBM + 32];
  float (&s1)[kBM + 32];
};

// One output tile: rows [m0, m0 + 256) x columns [n0, n0 + 32 kCols), kCols = 8 (256
// columns, wave tiles 64 x 128) or 4 (128 columns, wave tiles 64 x 64).
template <int kCols>
__device__ __forceinline__ void prefill_tile(const uint8_t* __restrict__ a_q,
                                             const float* __restrict__ a_scale,
                                             const uint8_t* __restrict__ w_q,
                                             const float* __restrict__ w_scale,
                                             uint16_t* __restrict__ out, int m, int n, int k,
                                             int ldc, int vec_out, int m0, int n0,
                                             const Stages& st) {
  constexpr int kWaveCols = 16 * kCols;   // columns per wave
  constexpr int kTileCols = 2 * kWaveCols;
  constexpr int kBBlocks = kTileCols / 8 / 8;  // 1 KB weight copy blocks per wave per group
  const int t = int(threadIdx.x), lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;  // rows 64 wm .., columns kWaveCols * wn ..
  const int groups = k >> 7;

  const __amdgpu_buffer_rsrc_t ra_rsrc = tile_rsrc(a_q, m0, m, k, kBM);
  const __amdgpu_buffer_rsrc_t rb_rsrc = tile_rsrc(w_q, n0, n, k, kTileCols);
  const __amdgpu_buffer_rsrc_t none_rsrc = tile_rsrc(a_q, 0, 0, k, 0);
  // 1 KB copy blocks (8 rows each): wave w fills blocks w + 8q of each operand; lane L of
  // block b loads row 8b + L/8, chunk (L % 8) ^ (L / 8) ^ (b & 1), which the swizzle below
  // places at byte b * 1024 + 16 L
  int voff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int b = wave + 8 * q, r = 8 * b + (lane >> 3);
    voff[q] = r * k + (((lane & 7) ^ (lane >> 3) ^ (b & 1)) << 4);
  }
  // activation scales: lane L of wave w copies row 32 w + L into slot 32 w + L (lanes
  // 32..63 repeat what wave w + 1 copies: same values, same slots; no branch)
  // lanes 32 and 33 of wave 7 (whose slots 256.. lie past the tile's rows) copy the weight
  // block scales of the two column halves instead, into slots 256 and 257
  const float* gsp = a_scale + int64_t(min(m0 + 32 * wave + lane, m - 1)) * groups;
  if (wave == 7 && (lane == 32 || lane == 33))
    gsp = w_scale + int64_t(min((n0 + kWaveCols * (lane - 32)) >> 7, (n >> 7) - 1)) * groups;

  // The copies of group g; outside [0, groups) they read a zero-size buffer (zeros written,
  // no memory traffic) and repeat a valid scale.  Every copy is unconditional: a branch
  // here would split the step and let the compiler sink its FMAs past the next barrier.
  auto copy_group = [&](uint8_t* sa, uint8_t* sb, float* ss, int g) {
    const bool live = g >= 0 && g < groups;
    const __amdgpu_buffer_rsrc_t ra = live ? ra_rsrc : none_rsrc;
    const __amdgpu_buffer_rsrc_t rb = live ? rb_rsrc : none_rsrc;
    const int goff = live ? g * 128 : 0;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(sa + (wave + 8 * q) * 1024), 16,
                                               voff[q], goff, 0, 0);
#pragma unroll
    for (int q = 0; q < kBBlocks; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(sb + (wave + 8 * q) * 1024), 16,
                                               voff[q], goff, 0, 0);
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void*)(gsp + min(max(g, 0), groups - 1)),
        (lds_void*)(ss + 32 * wave), 4, 0, 0);
  };

  v4f acc[4][kCols];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < kCols; ++c) acc[i][c] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // Staged 128-byte row r keeps its 16-byte chunk c at slot c ^ (r & 7) ^ (bit 3 of r): an
  // operand read takes one chunk from 16 consecutive rows per 16 lanes, which land on 16
  // distinct bank groups.  Fragment row 64 wm + 16 i + orow (or kWaveCols wn + 16 c + orow)
  // has the swizzle of row orow, so every read is one of four lane offsets plus a constant.
  const int orow = lane & 15, oh = lane >> 4;
  const int sw = (orow & 7) ^ ((orow >> 3) & 1);
  const int a_lo = (wm * 64 + orow) * 128 + (((2 * oh) ^ sw) << 4);
  const int a_hi = (wm * 64 + orow) * 128 + (((2 * oh + 1) ^ sw) << 4);
  const int b_lo = (wn * kWaveCols + orow) * 128 + (((2 * oh) ^ sw) << 4);
  const int b_hi = (wn * kWaveCols + orow) * 128 + (((2 * oh + 1) ^ sw) << 4);
  const int s_off = (wm * 64 + oh * 4) * 4;
  auto ld32 = [&](const uint8_t* p, int lo, int hi) {
    const v4u x = *reinterpret_cast<const v4u*>(p + lo);
    const v4u y = *reinterpret_cast<const v4u*>(p + hi);
    v8i r;
    r[0] = int(x[0]); r[1] = int(x[1]); r[2] = int(x[2]); r[3] = int(x[3]);
    r[4] = int(y[0]); r[5] = int(y[1]); r[6] = int(y[2]); r[7] = int(y[3]);
    return r;
  };

  // Group g from stage (sa, sb, ss); the copies of group g + 1 go to (na, nbs, ns), which
  // held group g - 1 (read by everyone before the barrier).
  auto step = [&](int g, const uint8_t* sa, const uint8_t* sb, const float* ss, uint8_t* na,
                  uint8_t* nbs, float* ns) {
    __syncthreads();  // everyone's copies of group g landed (the fence drains them)
    copy_group(na, nbs, ns, g + 1);
    // Column 0 starts once B_0, A_0 and A_1 are in: each later fragment is read one MFMA
    // ahead of its use, the scales last (their first use is column 0's FMAs, in column 1).
    v8i af[4];
    float4 as[4];
    v4f pcur[4], pprev[4];
    v8i bcur = ld32(sb, b_lo, b_hi);
    af[0] = ld32(sa, a_lo, a_hi);
    af[1] = ld32(sa + 2048, a_lo, a_hi);
    __builtin_amdgcn_sched_barrier(0);
    pcur[0] = mfma_group(af[0], bcur);
    __builtin_amdgcn_sched_barrier(0);
    af[2] = ld32(sa + 2 * 2048, a_lo, a_hi);
    __builtin_amdgcn_sched_barrier(0);
    pcur[1] = mfma_group(af[1], bcur);
    __builtin_amdgcn_sched_barrier(0);
    af[3] = ld32(sa + 3 * 2048, a_lo, a_hi);
    __builtin_amdgcn_sched_barrier(0);
    pcur[2] = mfma_group(af[2], bcur);
    __builtin_amdgcn_sched_barrier(0);
    v8i bnxt = ld32(sb + 2048, b_lo, b_hi);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      as[i] = *reinterpret_cast<const float4*>(reinterpret_cast<const uint8_t*>(ss) + s_off +
                                               i * 64);
    const float ws = ss[kBM + wn];
    __builtin_amdgcn_sched_barrier(0);
    pcur[3] = mfma_group(af[3], bcur);
    __builtin_amdgcn_sched_barrier(0);
    float f[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i][0] = as[i].x * ws; f[i][1] = as[i].y * ws; f[i][2] = as[i].z * ws;
      f[i][3] = as[i].w * ws;
      pprev[i] = pcur[i];
    }
    bcur = bnxt;
#pragma unroll
    for (int c = 1; c <= kCols; ++c) {
      bnxt = bcur;
      if (c + 1 < kCols) bnxt = ld32(sb + (c + 1) * 2048, b_lo, b_hi);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (c < kCols) pcur[i] = mfma_group(af[i], bcur);
        acc[i][c - 1][0] = __builtin_fmaf(pprev[i][0], f[i][0], acc[i][c - 1][0]);
        acc[i][c - 1][1] = __builtin_fmaf(pprev[i][1], f[i][1], acc[i][c - 1][1]);
        acc[i][c - 1][2] = __builtin_fmaf(pprev[i][2], f[i][2], acc[i][c - 1][2]);
        acc[i][c - 1][3] = __builtin_fmaf(pprev[i][3], f[i][3], acc[i][c - 1][3]);
      }
      if (c < kCols) {  // MFMA, its neighbour's four FMAs, MFMA, ...
        if (c + 1 < kCols) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (c == 1)
            __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
          else
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4; ++i) pprev[i] = pcur[i];
      bcur = bnxt;
    }
  };

  // An odd group count starts with one step over a zero group, so that steps come in
  // pairs and each step's stage is fixed at compile time.
  const int odd = groups & 1;
  copy_group(st.a0, st.b0, st.s0, -odd);
  for (int g = -odd; g < groups; g += 2) {
    step(g, st.a0, st.b0, st.s0, st.a1, st.b1, st.s1);
    step(g + 1, st.a1, st.b1, st.s1, st.a0, st.b0, st.s0);
  }
  __syncthreads();  // every copy landed and every wave is done reading the stages

  // output rows 64 s .. 64 s + 63 are staged in operand array s
  auto slab = [&](int s) -> uint8_t* {
    return s == 0 ? st.a0 : s == 1 ? st.a1 : s == 2 ? st.b0 : st.b1;
  };
  {
    uint16_t* sc = reinterpret_cast<uint16_t*>(slab(wm));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < kCols; ++c)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = i * 16 + oh * 4 + j;
          const int col = wn * kWaveCols + c * 16 + (lane & 15);
          sc[r * kCPitch + col] = f32_to_bf16_rne(acc[i][c][j]);
        }
  }
  __syncthreads();
  constexpr int kRowChunks = kTileCols / 8;  // 16-byte chunks per output row
#pragma unroll 4
  for (int q = 0; q < kBM * kRowChunks / kThreads; ++q) {
    const int ch = t + kThreads * q, r = ch / kRowChunks, cc = (ch % kRowChunks) * 8;
    const int gm = m0 + r, gn = n0 + cc;
    if (gm < m && gn < n) {
      const uint16_t* src =
          reinterpret_cast<const uint16_t*>(slab(r >> 6)) + (r & 63) * kCPitch + cc;
      uint16_t* dst = out + int64_t(gm) * ldc + gn;
      if (vec_out) {
        *reinterpret_cast<v4u*>(dst) = *reinterpret_cast<const v4u*>(src);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) dst[e] = src[e];
      }
    }
  }
}

// Work item b: items [0, n_full) are whole tiles, the rest are the two halves of each of
// the last tiles of the walk order.
__global__ __launch_bounds__(kThreads, 1) void w8a8_prefill_kernel(
    const uint8_t* __restrict__ a_q, const float* __restrict__ a_scale,
    const uint8_t* __restrict__ w_q, const float* __restrict__ w_scale,
    uint16_t* __restrict__ out, int m, int n, int k, int ldc, int tiles_m, int tiles_n,
    int n_full, int vec_out) {
  __shared__ __attribute__((aligned(16))) uint8_t a0[kSlab], a1[kSlab], b0[kSlab], b1[kSlab];
  __shared__ __attribute__((aligned(16))) float s0[kBM + 32], s1[kBM + 32];
  const Stages st{a0, a1, b0, b1, s0, s1};

  int item = int(blockIdx.x), tile = item, half = -1;
  if (item < n_full) {
    const int even = n_full - n_full % kXcds;
    if (item < even) tile = (item % kXcds) * (even / kXcds) + item / kXcds;
  } else {
    tile = n_full + (item - n_full) / 2;
    half = (item - n_full) & 1;
  }
  const int band = kGroupM * tiles_n;
  const int first_m = (tile / band) * kGroupM;
  const int band_m = min(kGroupM, tiles_m - first_m);
  const int tm = first_m + (tile % band) % band_m;
  const int tn = (tile % band) / band_m;
  const int m0 = tm * kBM, n0 = tn * kBN;
  if (half < 0)
    prefill_tile<8>(a_q, a_scale, w_q, w_scale, out, m, n, k, ldc, vec_out, m0, n0, st);
  else
    prefill_tile<4>(a_q, a_scale, w_q, w_scale, out, m, n, k, ldc, vec_out, m0, n0 + 128 * half,
                    st);
}

}  // namespace tile256

namespace tile128 {

constexpr int kBM = 128, kBN = 128, kThreads = 256;
constexpr int kAStage = kBM * 128;        // one group of the activation tile (bytes)
constexpr int kBStage = kBN * 128;        // one group of the weight tile
constexpr int kStage = kAStage + kBStage;
constexpr int kCPitch = kBN + 8;          // bf16 elements per staged output row
constexpr int kGroupM = 8;                // row tiles per column tile in the walk order
static_assert(kBM * kCPitch * 2 <= 2 * kStage, "output staging reuses the operand stages");

// LDS byte offset of 16-byte chunk c (0..7) of staged 128-byte row r: the chunk sits at
// slot c ^ (r & 7) ^ (bit 3 of r).  An MFMA operand read takes one chunk index from 16
// consecutive rows per 16 lanes: those 16 rows land on 16 distinct 16-byte bank groups of
// the 256-byte bank row, so the read is conflict-free.
__device__ __forceinline__ int lds_chunk(int r, int c) {
  return r * 128 + ((c ^ (r & 7) ^ ((r >> 3) & 1)) << 4);
}

// 32 operand bytes of row r: chunks 2h and 2h + 1.
__device__ __forceinline__ v8i lds_load32(const uint8_t* base, int row, int h) {
  const v4u x = *reinterpret_cast<const v4u*>(base + lds_chunk(row, 2 * h));
  const v4u y = *reinterpret_cast<const v4u*>(base + lds_chunk(row, 2 * h + 1));
  v8i r;
  r[0] = int(x[0]); r[1] = int(x[1]); r[2] = int(x[2]); r[3] = int(x[3]);
  r[4] = int(y[0]); r[5] = int(y[1]); r[6] = int(y[2]); r[7] = int(y[3]);
  return r;
}

// Operand tiles are copied global -> LDS by the buffer unit itself (buffer_load ... lds):
// no staging registers and no LDS store instructions.  A wave's copy instruction fills one
// contiguous 1 KB block of LDS, lane L writing bytes [16L, 16L + 16); so lane L of block b
// loads the global chunk that the swizzle puts at row 8b + L/8, slot L % 8.  Per group: wait
// for this wave's copies, one barrier, read every operand fragment of the group, start the
// copies of the next group into the other buffer, then multiply -- the copies run under
// the MFMAs.  (The copies are issued only after the group's LDS reads: the compiler orders
// every LDS read after all outstanding copies, so a copy issued earlier would stall them.)
__global__ __launch_bounds__(kThreads, 2) void w8a8_prefill_small_kernel(
    const uint8_t* __restrict__ a_q, const float* __restrict__ a_scale,
    const uint8_t* __restrict__ w_q, const float* __restrict__ w_scale,
    uint16_t* __restrict__ out, int m, int n, int k, int ldc, int tiles_m, int tiles_n,
    int vec_out) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStage];
  __shared__ __attribute__((aligned(16))) float s_as[2][kBM];

  const int nblk = tiles_m * tiles_n;
  int bid = int(blockIdx.x);
  const int even = nblk - nblk % kXcds;
  if (bid < even) bid = (bid % kXcds) * (even / kXcds) + bid / kXcds;
  const int band = kGroupM * tiles_n;
  const int first_m = (bid / band) * kGroupM;
  const int band_m = min(kGroupM, tiles_m - first_m);
  const int tm = first_m + (bid % band) % band_m;
  const int tn = (bid % band) / band_m;
  const int m0 = tm * kBM, n0 = tn * kBN;

  const int t = int(threadIdx.x), lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int groups = k >> 7;

  const __amdgpu_buffer_rsrc_t ra_rsrc = tile_rsrc(a_q, m0, m, k, kBM);
  const __amdgpu_buffer_rsrc_t rb_rsrc = tile_rsrc(w_q, n0, n, k, kBN);
  // wave w fills blocks b = w + 4q (q < 4) of each operand stage: rows 8b .. 8b + 7
  int voff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int b = wave + 4 * q, r = 8 * b + (lane >> 3);
    const int c = (lane & 7) ^ (lane >> 3) ^ (b & 1);  // lds_chunk(r, c) == b*1024 + 16*lane
    voff[q] = r * k + c * 16;
  }
  // activation scales: wave w copies rows 32w .. 32w + 31 of column g (lanes 0..31)
  const float* gsp = a_scale + int64_t(min(m0 + 32 * wave + (lane & 31), m - 1)) * groups;
  const_float* wsp = (const_float*)(w_scale + int64_t(n0 >> 7) * groups);

  auto copy_group = [&](int buf, int g) {
    uint8_t* base = lds + buf * kStage;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra_rsrc, (lds_void*)(base + (wave + 4 * q) * 1024),
                                               16, voff[q], g * 128, 0, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb_rsrc, (lds_void*)(base + kAStage + (wave + 4 * q) * 1024), 16, voff[q], g * 128,
          0, 0);
    if (lane < 32)
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(gsp + g),
                                       (lds_void*)(&s_as[buf][32 * wave]), 4, 0, 0);
  };

  v4f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[i][c] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  const int orow = lane & 15, oh = lane >> 4;
  copy_group(0, 0);
  for (int g = 0; g < groups; ++g) {
    const int buf = g & 1;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies of group g landed
    __syncthreads();                     // ... and everyone's; buffer buf^1 is free again
    const uint8_t* sa = lds + buf * kStage;
    const uint8_t* sb = sa + kAStage;
    const float ws = wsp[g];
    v8i af[4], bf[4];
    float4 as[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      af[i] = lds_load32(sa, wm * 64 + i * 16 + orow, oh);
      as[i] = *reinterpret_cast<const float4*>(&s_as[buf][wm * 64 + i * 16 + oh * 4]);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) bf[c] = lds_load32(sb, wn * 64 + c * 16 + orow, oh);
    if (g + 1 < groups) copy_group(buf ^ 1, g + 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float f0 = as[i].x * ws, f1 = as[i].y * ws, f2 = as[i].z * ws, f3 = as[i].w * ws;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const v4f p = mfma_group(af[i], bf[c]);
        acc[i][c][0] = __builtin_fmaf(p[0], f0, acc[i][c][0]);
        acc[i][c][1] = __builtin_fmaf(p[1], f1, acc[i][c][1]);
        acc[i][c][2] = __builtin_fmaf(p[2], f2, acc[i][c][2]);
        acc[i][c][3] = __builtin_fmaf(p[3], f3, acc[i][c][3]);
      }
    }
  }
  __syncthreads();  // every wave is done reading the last stage before it is reused

  uint16_t* sc = reinterpret_cast<uint16_t*>(lds);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = wm * 64 + i * 16 + oh * 4 + j;
        const int col = wn * 64 + c * 16 + (lane & 15);
        sc[r * kCPitch + col] = f32_to_bf16_rne(acc[i][c][j]);
      }
  __syncthreads();
#pragma unroll 4
  for (int q = 0; q < kBM * kBN / 8 / kThreads; ++q) {
    const int ch = t + kThreads * q, r = ch >> 4, cc = (ch & 15) * 8;
    const int gm = m0 + r, gn = n0 + cc;
    if (gm < m && gn < n) {
      const uint16_t* src = sc + r * kCPitch + cc;
      uint16_t* dst = out + int64_t(gm) * ldc + gn;
      if (vec_out) {
        *reinterpret_cast<v4u*>(dst) = *reinterpret_cast<const v4u*>(src);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) dst[e] = src[e];
      }
    }
  }
}

}  // namespace tile128

}  // namespace
}  // namespace fp8q

using namespace fp8q;

extern "C" int w8a8_block_gemm_prefill(const uint8_t* a_q, const float* a_scale,
                                       const uint8_t* w_q, const float* w_scale, uint16_t* out,
                                       int32_t m, int32_t n, int32_t k, int32_t ldc,
                                       hipStream_t stream) {
  if (m < 1 || n <= 0 || n % 128 != 0 || k <= 0 || k % 128 != 0 || ldc < n) return FP8Q_EINVAL;
  if (!a_q || !a_scale || !w_q || !w_scale || !out) return FP8Q_ENULL;
  if (!aligned(a_q, 16) || !aligned(w_q, 16) || !aligned(a_scale, 4) || !aligned(w_scale, 4) ||
      !aligned(out, 2))
    return FP8Q_EALIGN;
  // buffer offsets within one 128-row tile are 32-bit
  if (int64_t(128) * k > 0x7FFFFFFF) return FP8Q_EINVAL;
  const int vec_out = (ldc % 8 == 0 && aligned(out, 16)) ? 1 : 0;
  const int64_t cus = num_cus();
  const int64_t big_m = (int64_t(m) + 255) / 256, big_n = (int64_t(n) + 255) / 256;
  const int64_t big = big_m * big_n;
  if (2 * big >= cus && int64_t(256) * k <= 0x7FFFFFFF && big <= 0x3FFFFFFF) {
    // one workgroup per CU: split the tiles of a last round that would leave half the CUs
    // idle
    const int64_t tail = big % cus;
    const int64_t split = (tail != 0 && 2 * tail <= cus) ? tail : 0;
    const int64_t n_full = big - split;
    launch(tile256::w8a8_prefill_kernel, dim3(unsigned(n_full + 2 * split)),
           dim3(tile256::kThreads), 0, stream, a_q, a_scale, w_q, w_scale, out, m, n, k, ldc,
           int(big_m), int(big_n), int(n_full), vec_out);
    return launch_status();
  }
  const int64_t tiles_m = (int64_t(m) + 127) / 128, tiles_n = (int64_t(n) + 127) / 128;
  if (tiles_m * tiles_n > 0x7FFFFFFF) return FP8Q_EINVAL;
  launch(tile128::w8a8_prefill_small_kernel, dim3(unsigned(tiles_m * tiles_n)),
         dim3(tile128::kThreads), 0, stream, a_q, a_scale, w_q, w_scale, out, m, n, k, ldc,
         int(tiles_m), int(tiles_n), vec_out);
  return launch_status();
}
