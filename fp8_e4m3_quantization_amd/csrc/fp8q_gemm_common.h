// fp8q_gemm_common.h -- pieces shared by the persistent decode GEMM kernels (W8A8 and
// W8A16): MFMA operand vector types, the projection set one launch walks, the strip
// lookup, buffer descriptors for the weight stream and the LDS-only barrier.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8q_device.h"

namespace fp8q {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kMaxProj = 8;  // projections of one activation in one launch
constexpr int kPWaves = 8;   // waves of a persistent workgroup (one workgroup per CU)

// Several projections that read the same activation: output strips of 16 columns are
// numbered across them in order.
struct ProjSet {
  const uint8_t* w[kMaxProj];
  const float* ws[kMaxProj];
  uint16_t* out[kMaxProj];
  int ldc[kMaxProj];
  int strip_end[kMaxProj];  // cumulative strip count after projection p
  int count;
};

// strip s -> (projection, first column); uniform across the workgroup
__device__ __forceinline__ void locate_strip(const ProjSet& ps, int s, int* p_out, int* n0) {
  int p = 0;
  while (p + 1 < ps.count && s >= ps.strip_end[p]) ++p;
  *p_out = p;
  *n0 = (s - (p ? ps.strip_end[p - 1] : 0)) * 16;
}

// s_waitcnt lgkmcnt(0) + s_barrier: orders the LDS partials without waiting on the
// weight prefetches that are still in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt untouched
  __builtin_amdgcn_s_barrier();
}

// Weight loads go through a buffer descriptor per strip (base = the strip's first row,
// 16*k bytes).  A strip past the end gets a zero-size descriptor: its loads return zeros
// without touching memory, so every prefetch is issued unconditionally and the compiler
// tracks the in-order load counter exactly (no branch around any load).
constexpr uint32_t kBufferDword3 = 0x00020000;  // raw 32-bit buffer format (gfx9 family)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_strip_rsrc(const uint8_t* base, int k,
                                                                  bool valid, int rows = 16) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, valid ? rows * k : 0,
                                           kBufferDword3);
}

// ---------------------------------------------------------------------------------
// Work items of a persistent launch.  Strips [0, half_from) are whole items; every later
// strip is two items of 8 columns (item half_from + 2 (s - half_from) + h covers columns
// 8h .. 8h + 7 of strip s).  When the strips leave a last round at most half full, its
// strips are halved so that every workgroup takes one half: each then streams the same
// bytes, instead of half the workgroups streaming a whole extra strip while the rest idle.
// A half item reads its 8 weight rows through a descriptor 8 rows long, so the other 8
// rows of the MFMA's weight operand read as zeros and only the item's own 8 output
// columns are stored: the products of the stored columns are the whole strip's.
struct StripItem {
  int strip;  // strip index
  int col0;   // first column of the item within the strip (0 or 8)
  int cols;   // 16, or 8 for a half
};
__device__ __forceinline__ StripItem strip_item(int item, int half_from) {
  if (item < half_from) return StripItem{item, 0, 16};
  const int h = item - half_from;
  return StripItem{half_from + (h >> 1), 8 * (h & 1), 8};
}

// First halved strip for `strips` strips over `grid` workgroups (strips: none halved).
__host__ __device__ inline int halved_from(int strips, int grid) {
  const int rest = strips % grid;
  return (rest != 0 && 2 * rest <= grid) ? strips - rest : strips;
}
__host__ __device__ inline int item_count(int strips, int half_from) { return half_from + 2 * (strips - half_from); }

// Weight block scales are read-only for the whole launch and uniform per wave: reading
// them through the constant address space makes them scalar loads (counted apart from
// the vector weight loads, so waiting for a scale never drains the weight prefetch).
typedef const __attribute__((address_space(4))) float const_float;

// 32 bytes at byte offset off of a buffer, as eight dwords (two 16-byte loads).
template <int kAux>
__device__ __forceinline__ v8i buffer_load32(__amdgpu_buffer_rsrc_t r, int off) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAux);
  const v4u y = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, kAux);
  v8i o;
  o[0] = int(x[0]); o[1] = int(x[1]); o[2] = int(x[2]); o[3] = int(x[3]);
  o[4] = int(y[0]); o[5] = int(y[1]); o[6] = int(y[2]); o[7] = int(y[3]);
  return o;
}

// ---------------------------------------------------------------------------------
// Where a workgroup starts.  Block b walks strips first, first + grid, ...  Workgroups are
// dealt to the chip's 8 XCDs round robin (block b runs on XCD b % 8), so with the plain
// order first = b the 16-column strips of one 128-column output block land on 8 different
// XCDs, and each XCD's L2 holds only 32-byte pieces of every output row.  When the grid is
// a multiple of 64, blocks are permuted so that every run of 8 adjacent strips belongs to
// the 8 blocks of a single XCD (the strips of a run are processed at the same time, so
// that L2 gathers whole output lines before writing them back).
__device__ __forceinline__ int first_strip(int b, int grid) {
  if (grid % 64 != 0) return b;
  const int xcd = b & 7, k = b >> 3;     // k-th block of XCD xcd
  return (((k >> 3) * 8 + xcd) << 3) | (k & 7);
}

// ---------------------------------------------------------------------------------
// Activation fragments through LDS.  The MFMA operand layout gives lane l row (l & 15) and
// 32 consecutive k of a 128-wide group; loaded straight from global memory every load
// instruction would touch 16 rows in partial lines, while every workgroup on the chip
// reads the same activation at the same time.  Instead a wave reads a group's 16-row
// tile row-major (16 bytes per lane, whole rows per instruction), passes it through a
// wave-private LDS tile and reads its own fragment back.  The tile is swizzled so that
// the row-major writes and the fragment reads are both free of bank conflicts.  A wave's
// LDS operations complete in program order, so the tile is reused group after group with
// no barrier.
typedef unsigned v4u __attribute__((ext_vector_type(4)));

template <int kChunks>  // 16-byte chunks per tile row: 8 (E4M3 codes) or 16 (bf16)
struct ActTile {
  static_assert(kChunks == 8 || kChunks == 16, "tile rows of 128 or 256 bytes");
  static constexpr int kLoads = 16 * kChunks / 64;  // 16-byte loads per lane per tile
  static constexpr int kUints = 16 * kChunks;       // tile size in 16-byte chunks
  __device__ static int row(int t, int lane) { return t * (64 / kChunks) + lane / kChunks; }
  __device__ static int slot(int r, int c) {
    return kChunks == 8 ? (c ^ (r & 7) ^ ((r >> 3) & 1)) : (c ^ r);
  }
  // Global reads of one tile: `group` is the group's first byte in row 0, rows are `pitch`
  // bytes apart; rows >= m repeat row m - 1 (in bounds; their fragments are never used).
  __device__ static void load(const uint8_t* group, int64_t pitch, int m, int lane,
                              v4u (&out)[kLoads]) {
#pragma unroll
    for (int t = 0; t < kLoads; ++t) {
      const int r = min(row(t, lane), m - 1);
      out[t] = *reinterpret_cast<const v4u*>(group + r * pitch + 16 * (lane % kChunks));
    }
  }
  // Tile -> LDS, then the lane's kFrag chunks first_chunk, first_chunk + 1, ... of row
  // (lane & 15).
  template <int kFrag>
  __device__ static void exchange(uint4* tile, const v4u (&in)[kLoads], int lane,
                                  int first_chunk, uint4 (&frag)[kFrag]) {
#pragma unroll
    for (int t = 0; t < kLoads; ++t) {
      const int r = row(t, lane);
      tile[r * kChunks + slot(r, lane % kChunks)] = make_uint4(in[t][0], in[t][1], in[t][2], in[t][3]);
    }
    const int r = lane & 15;
#pragma unroll
    for (int i = 0; i < kFrag; ++i) frag[i] = tile[r * kChunks + slot(r, first_chunk + i)];
  }
};

// ---------------------------------------------------------------------------------
// The W8A16 tier's weight operand: E4M3 codes widened to bf16 for v_mfma_f32_16x16x32_bf16.
typedef __bf16 v8bf16 __attribute__((ext_vector_type(8)));

// Two E4M3 codes (bytes 0,1 or 2,3 of w) -> two bf16 in one word: the binary32 decode is
// exact and its top half is the bf16 value (no rounding: three mantissa bits).
template <bool kHigh>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  const float2 f = e4m3x2_to_f32<kHigh>(w);
  return __builtin_amdgcn_perm(__float_as_uint(f.y), __float_as_uint(f.x), 0x07060302u);
}

// Eight codes (two dwords) -> the eight bf16 of one MFMA operand, in k order.
__device__ __forceinline__ v8bf16 widen8(uint32_t lo, uint32_t hi) {
  const uint4 r = make_uint4(e4m3x2_to_bf16x2<false>(lo), e4m3x2_to_bf16x2<true>(lo),
                             e4m3x2_to_bf16x2<false>(hi), e4m3x2_to_bf16x2<true>(hi));
  return __builtin_bit_cast(v8bf16, r);
}

// The W8A16 tier over a projection set in the staged form (fp8q_gemm.hip): k a multiple of
// 1024, k <= 8192, 1 <= m <= 4.
int run_w8a16_staged(const uint16_t* a, const ProjSet& ps, int m, int k, hipStream_t stream);

}  // namespace fp8q
