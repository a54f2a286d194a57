// fp8q_gemm_prefill.hip -- block-scaled W8A8 GEMM for prefill widths (hundreds to thousands
// of activation rows): the dense, MFMA-bound form of the same arithmetic as the decode GEMM.
//
// fp8_residency.rs page, DenseFp8Inputs::w8a8_kernels (the W8A8 prefill arm is the
// per-token group quantizer followed by a block-scaled FP8 GEMM); fp8_act_quant.rs page,
// module doc (a 4593-token prefill); dispatch_proj_decode.rs page, module doc NUMERICS
// (E4M3 activations with per-token 1x128 FP32 scales times E4M3 weights with 128x128 FP32
// block scales, FP32 epilogue).
//
// Tiling for gfx950: a 256-thread workgroup owns a 128 x 128 output tile and walks K one
// 128-wide group at a time, two workgroups per CU.  Each step holds the group's 128 x 128
// activation and weight codes in LDS (double-buffered).  Wave (wm, wn) of the 2 x 2 grid
// owns 64 x 64 of the tile: 4 x 4 tiles of v_mfma_f32_16x16x128_f8f6f4, one instruction per
// tile per group, so every instruction's result is one group's partial and takes its scale
// a_scale[row, g] * w_scale[col/128, g] in one FMA per element.  The epilogue stages the bf16
// tile through LDS and writes it with 16-byte row-contiguous stores.  Workgroups are
// ordered so that concurrently running ones share operand tiles: 8 consecutive row tiles
// per column tile, and each XCD (workgroup ids are dealt to the 8 XCDs round-robin) takes a
// contiguous stretch of that order for its own L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8q.h"
#include "fp8q_gemm_common.h"
#include "fp8q_launch.h"
#include "fp8q_math.h"

#pragma clang fp contract(off)

namespace fp8q {
namespace {

constexpr int kBM = 128, kBN = 128, kThreads = 256;
constexpr int kAStage = kBM * 128;        // one group of the activation tile (bytes)
constexpr int kBStage = kBN * 128;        // one group of the weight tile
constexpr int kStage = kAStage + kBStage;
constexpr int kCPitch = kBN + 8;          // bf16 elements per staged output row
#ifndef FP8Q_PREFILL_GROUPM
#define FP8Q_PREFILL_GROUPM 8
#endif
constexpr int kGroupM = FP8Q_PREFILL_GROUPM;  // row tiles per column tile in the walk order
constexpr int kXcds = 8;
static_assert(kBM * kCPitch * 2 <= 2 * kStage, "output staging reuses the operand stages");

typedef unsigned v4u __attribute__((ext_vector_type(4)));

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

// E4M3 x E4M3 -> FP32 over one 128-wide K-group of a 16 x 16 tile (no scaling).
__device__ __forceinline__ v4f mfma_group(v8i a, v8i b) {
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// Buffer descriptor over rows [r0, rows) of a [rows, k] byte matrix: reads past the last
// row return zeros without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* base, int r0, int rows,
                                                            int k) {
  const int valid = rows - r0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base + int64_t(r0) * k), 0,
                                           valid > 0 ? valid * k : 0, kBufferDword3);
}

// Operand tiles are copied global -> LDS by the buffer unit itself (buffer_load ... lds):
// no staging registers and no LDS store instructions.  A wave's copy instruction fills one
// contiguous 1 KB block of LDS, lane L writing bytes [16L, 16L + 16); so lane L of block b
// loads the global chunk that the swizzle puts at row 8b + L/8, slot L % 8.  Per group: wait
// for this wave's copies, one barrier, read every operand fragment of the group, start the
// copies of the next group into the other buffer, then multiply -- the copies run under
// the MFMAs.  (The copies are issued only after the group's LDS reads: the compiler orders
// every LDS read after all outstanding copies, so a copy issued earlier would stall them.)
__global__ __launch_bounds__(kThreads, 2) void w8a8_prefill_kernel(
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

  const __amdgpu_buffer_rsrc_t ra_rsrc = tile_rsrc(a_q, m0, m, k);
  const __amdgpu_buffer_rsrc_t rb_rsrc = tile_rsrc(w_q, n0, n, k);
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

  typedef __attribute__((address_space(3))) void lds_void;
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
  const int64_t tiles_m = (int64_t(m) + kBM - 1) / kBM;
  const int64_t tiles_n = (int64_t(n) + kBN - 1) / kBN;
  if (tiles_m * tiles_n > 0x7FFFFFFF) return FP8Q_EINVAL;
  // buffer offsets within one 128-row tile are 32-bit
  if (int64_t(kBM) * k > 0x7FFFFFFF) return FP8Q_EINVAL;
  const int vec_out = (ldc % 8 == 0 && aligned(out, 16)) ? 1 : 0;
  launch(w8a8_prefill_kernel, dim3(unsigned(tiles_m * tiles_n)), dim3(kThreads), 0, stream,
         a_q, a_scale, w_q, w_scale, out, m, n, k, ldc, int(tiles_m), int(tiles_n), vec_out);
  return launch_status();
}
