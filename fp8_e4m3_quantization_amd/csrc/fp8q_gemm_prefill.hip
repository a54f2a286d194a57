// fp8q_gemm_prefill.hip -- block-scaled W8A8 GEMM for prefill widths (hundreds to thousands
// of activation rows): the dense, MFMA-bound form of the same arithmetic as the decode GEMM.
//
// fp8_residency.rs page, DenseFp8Inputs::w8a8_kernels (the W8A8 prefill arm is the
// per-token group quantizer followed by a block-scaled FP8 GEMM); fp8_act_quant.rs page,
// module doc (a 4593-token prefill); dispatch_proj_decode.rs page, module doc NUMERICS
// (E4M3 activations with per-token 1x128 FP32 scales times E4M3 weights with 128x128 FP32
// block scales, FP32 epilogue).
//
// The kernels walk K one 128-wide group at a time; one v_mfma_f32_16x16x128_f8f6f4 covers
// one group of a 16 x 16 output tile, so every instruction's result is one group's partial
// and takes its scale a_scale[row, g] * w_scale[col/128, g] in one FMA per element.  The
// operand tiles of each group are copied global -> LDS by the buffer unit itself
// (buffer_load ... lds: no staging registers, no LDS store instructions), the next groups'
// copies landing while the current group multiplies.
//
// tile256 (the large shapes): one 512-thread workgroup per CU owns a 256 x 256 output tile,
// wave (wm, wn) of the 4 x 2 grid 64 x 128 of it (4 x 8 MFMA tiles).  A 256 x 256 tile
// copies half the operand bytes per flop of a 128 x 128 one, which the copy path (the
// texture/address unit, about 70 % busy with 128 x 128 tiles) needs, and 64 x 128 per wave
// reads 0.75 KB of LDS per MFMA.  The column loop is software-pipelined: column c + 1's
// weight fragment is read and column c - 1's products are scaled while column c
// multiplies, one group of four FMAs between MFMAs; after each group's barrier only B_0
// and the first two activation fragments are read before the first MFMA, each later
// fragment an MFMA ahead of its use.  When the tile count leaves the last round of
// workgroups at most half full, each of those last tiles is split into two 256 x 128 halves
// (wave tiles 64 x 64): twice as many work items, each half as long.  Two forms:
//  - ring (group count a multiple of eight): five 32 KB LDS slots in rotation, each weight
//    tile copied two groups ahead and each activation tile one; the scales go to
//    registers (no LDS is left), the weight scale by a scalar load issued after the
//    step's last LDS read.  It hides the copies that miss L2 better than two stages.
//  - two_stage (any group count): two stages of both operand tiles and the scales (the
//    weight block scale rides in the activation-scale copy), one group ahead.
// Results are the same bit for bit: the same products, scaled and summed in the same order.
//
// tile128 (fewer than half a round of 256 x 256 tiles, e.g. a 1024-column projection or a
// short prefill): 256-thread workgroups, up to two per CU, each a 128 x 128 tile (2 x 2
// waves of 64 x 64).  With at most one tile per CU and a group count that is a multiple of
// eight it runs on the same five-slot ring (16 KB slots), else on two stages.
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

// ---------------------------------------------------------------------------------------
// Shared by the tiled kernels.  A wave tile is 64 rows x 16 kCols columns; the waves form a
// kWM x kWN grid (4 x 2: 256 x 256 or 256 x 128 tiles of 8 waves; 2 x 2: 128 x 128 tiles of
// 4 waves).

// Staged 128-byte operand row r keeps its 16-byte chunk c at slot c ^ (r & 7) ^ (bit 3 of
// r): an operand read takes one chunk from 16 consecutive rows per 16 lanes, which land on
// 16 distinct bank groups.  Fragment row 64 wm + 16 i + orow (or wave_cols wn + 16 c +
// orow) has the swizzle of row orow, so every read is one of four lane offsets plus a
// constant.  A 1 KB copy block (8 rows) is one copy instruction: lane L of block b loads
// row 8b + L/8, chunk (L % 8) ^ (L / 8) ^ (b & 1), which the swizzle places at byte
// b * 1024 + 16 L.
struct Frag {
  int a_lo, a_hi, b_lo, b_hi;
};
__device__ __forceinline__ Frag frag_offsets(int lane, int wm, int wn, int wave_cols) {
  const int orow = lane & 15, oh = lane >> 4;
  const int sw = (orow & 7) ^ ((orow >> 3) & 1);
  return {(wm * 64 + orow) * 128 + (((2 * oh) ^ sw) << 4),
          (wm * 64 + orow) * 128 + (((2 * oh + 1) ^ sw) << 4),
          (wn * wave_cols + orow) * 128 + (((2 * oh) ^ sw) << 4),
          (wn * wave_cols + orow) * 128 + (((2 * oh + 1) ^ sw) << 4)};
}

// The 32 operand bytes of one MFMA fragment: chunks at byte offsets lo and hi of p.
__device__ __forceinline__ v8i ld32(const uint8_t* p, int lo, int hi) {
  const v4u x = *reinterpret_cast<const v4u*>(p + lo);
  const v4u y = *reinterpret_cast<const v4u*>(p + hi);
  v8i r;
  r[0] = int(x[0]); r[1] = int(x[1]); r[2] = int(x[2]); r[3] = int(x[3]);
  r[4] = int(y[0]); r[5] = int(y[1]); r[6] = int(y[2]); r[7] = int(y[3]);
  return r;
}

// Each MFMA takes the weight fragment as its first operand, so its 16 x 16 result is the
// transposed tile: element j of lane (oh, orow) in row tile i is row 16 i + orow of the
// wave's 64 and column 4 oh + j of the 16 -- one activation scale per lane and row tile.
//
// The bf16 output tile is staged through kWM operand arrays (rows 64 s .. 64 s + 63 in
// array s at a pitch of one tile row; row r's 8-column blocks XOR-permuted by bits 0..3 of
// r, so that the 16 rows one 8-byte store instruction writes spread over the bank groups),
// then written out in 16-byte row pieces.  Called after a barrier that ends every operand
// read.
template <int kWM, int kWN, int kCols>
__device__ __forceinline__ void store_tile(const v4f (&acc)[4][kCols], uint8_t* s0, uint8_t* s1,
                                           uint8_t* s2, uint8_t* s3, uint16_t* __restrict__ out,
                                           int m, int n, int ldc, int vec_out, int m0, int n0) {
  constexpr int kWaveCols = 16 * kCols, kTileCols = kWN * kWaveCols;
  constexpr int kRows = 64 * kWM, kThreads = 64 * kWM * kWN;
  static_assert(kTileCols == 128 || kTileCols == 256, "the XOR permutation stays in the row");
  const int t = int(threadIdx.x), lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave / kWN, wn = wave % kWN;
  const int orow = lane & 15, oh = lane >> 4;
  auto slab = [&](int s) -> uint8_t* { return s == 0 ? s0 : s == 1 ? s1 : s == 2 ? s2 : s3; };
  {
    uint16_t* so = reinterpret_cast<uint16_t*>(slab(wm));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < kCols; ++c) {
        const int r = i * 16 + orow;
        const int col = (wn * kWaveCols + c * 16 + 4 * oh) ^ (orow << 3);
        const uint32_t lo = uint32_t(f32_to_bf16_rne(acc[i][c][0])) |
                            (uint32_t(f32_to_bf16_rne(acc[i][c][1])) << 16);
        const uint32_t hi = uint32_t(f32_to_bf16_rne(acc[i][c][2])) |
                            (uint32_t(f32_to_bf16_rne(acc[i][c][3])) << 16);
        *reinterpret_cast<uint2*>(so + r * kTileCols + col) = make_uint2(lo, hi);
      }
  }
  __syncthreads();
  constexpr int kRowChunks = kTileCols / 8;  // 16-byte chunks per output row
#pragma unroll 4
  for (int q = 0; q < kRows * kRowChunks / kThreads; ++q) {
    const int ch = t + kThreads * q, r = ch / kRowChunks, cc = (ch % kRowChunks) * 8;
    const int gm = m0 + r, gn = n0 + cc;
    if (gm < m && gn < n) {
      const uint16_t* src = reinterpret_cast<const uint16_t*>(slab(r >> 6)) +
                            (r & 63) * kTileCols + (cc ^ ((r & 15) << 3));
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

// ---------------------------------------------------------------------------------------
// Five-slot ring (group counts that are a multiple of eight).
//
// LDS: five slots, each a separate array (one operand tile of one group each; 5 x 32 KB =
// all 160 KB for the 256-row tiles, 5 x 16 KB for the 128 x 128 tiles).  Step g multiplies the activation tile and the weight tile of group g from two
// slots while the weight tile of group g + 1 lands in a third, and copies the activation
// tile of group g + 1 and the weight tile of group g + 2 into the two slots that group
// g - 1 used: a weight copy has two steps to land, an activation copy one.  The slots
// rotate with a period of eight steps: activation groups 8t + j sit in slots 4 3 4 1 4 0 4 2
// and weight groups in slots 0 1 2 0 3 2 1 3, so that the two activation groups and three
// weight groups of any step sit in five distinct slots.  Separate objects let the compiler
// see that a slot's operand reads never alias the copies landing in the others, so it keeps
// those copies in flight.  The scales take no LDS: each wave loads them into registers.
namespace ring {

// One group's scales as one lane holds them: the activation scale of row 64 wm + lane of
// the tile and the weight block scale of the wave's column block (uniform: a scalar).
struct Scales {
  float row, w;
};

template <int kBytes>
struct Slots {
  uint8_t (&x0)[kBytes];
  uint8_t (&x1)[kBytes];
  uint8_t (&x2)[kBytes];
  uint8_t (&x3)[kBytes];
  uint8_t (&x4)[kBytes];
};

// Where each of a step's kPieces copy pieces is dealt: the column before whose MFMAs it is
// issued, 0 meaning the first column (piece 0 ahead of its first MFMA, piece j after MFMA
// j - 1).  With eight columns: activation pieces two in column 0 and two before column 1,
// the row scales before column 2, weight block q before column 3 + q.  With four: the
// activation pieces after the first MFMAs, then the row scales and weight blocks one per
// column from column 1 while there are no more of them than columns, else spread over all
// of them.  The scalar load goes before the last column: every LDS read of the step is
// issued and waited for by then (scalar and LDS loads share a wait counter).  The barrier's
// wait count relies on the issue order: pieces go out in index order, so the row scales
// precede the weight blocks, the step's last vector loads.
template <int kCols, int kABlocks, int kPieces>
struct DealColumns {
  static constexpr int column(int j) {
    constexpr int kDealt = kPieces - 5;
    if (j == kPieces - 1) return kCols;
    if (kCols == 8) return j < 2 ? 0 : j < 4 ? 1 : j - 2;
    if (j < kABlocks) return 0;
    if (kDealt <= kCols) return j - 3;
    int c = 1;
    while (j >= 4 + c * kDealt / kCols) ++c;
    return c;
  }
  static constexpr bool valid() {
    if (kABlocks != 4) return false;
    for (int j = 0; j < kPieces; ++j) {
      if (column(j) < 0 || column(j) > kCols) return false;
      if (j > 0 && column(j) < column(j - 1)) return false;
      if (column(j) == 0 && j > 3) return false;  // three places after the first MFMAs
    }
    return column(0) == 0 && column(kPieces - 1) == kCols;
  }
};

// One output tile: rows [m0, m0 + 64 kWM) x columns [n0, n0 + 16 kWN kCols).
template <int kWM, int kWN, int kCols, int kBytes>
__device__ __forceinline__ void prefill_tile(const uint8_t* __restrict__ a_q,
                                             const float* __restrict__ a_scale,
                                             const uint8_t* __restrict__ w_q,
                                             const float* __restrict__ w_scale,
                                             uint16_t* __restrict__ out, int m, int n, int k,
                                             int ldc, int vec_out, int m0, int n0,
                                             const Slots<kBytes>& st) {
  constexpr int kWaves = kWM * kWN;
  constexpr int kRows = 64 * kWM;         // tile rows
  constexpr int kWaveCols = 16 * kCols;   // columns per wave
  constexpr int kTileCols = kWN * kWaveCols;
  static_assert(kRows * 128 <= kBytes && kTileCols * 128 <= kBytes, "a slot holds a tile");
  static_assert(kRows * kTileCols * 2 <= kWM * kBytes, "kWM slots hold the output tile");
  constexpr int kABlocks = kRows / 8 / kWaves;     // 1 KB activation copy blocks per wave
  constexpr int kBBlocks = kTileCols / 8 / kWaves;  // 1 KB weight copy blocks per wave
  static_assert(kABlocks >= 1 && kBBlocks >= 1 && kWaves % 2 == 0, "whole copy blocks");
  const int t = int(threadIdx.x), lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave / kWN, wn = wave % kWN;  // rows 64 wm .., columns kWaveCols * wn ..
  const int groups = k >> 7;

  const __amdgpu_buffer_rsrc_t ra_rsrc = tile_rsrc(a_q, m0, m, k, kRows);
  const __amdgpu_buffer_rsrc_t rb_rsrc = tile_rsrc(w_q, n0, n, k, kTileCols);
  const __amdgpu_buffer_rsrc_t none_rsrc = tile_rsrc(a_q, 0, 0, k, 0);
  // Scales: the wave's 64 activation rows (rows past m read as zeros) as a [rows, groups]
  // FP32 matrix, and the weight block row of its columns.  (readfirstlane: the descriptor
  // must be seen as uniform, or each load becomes a loop.)
  const int srow0 = __builtin_amdgcn_readfirstlane(min(m0 + 64 * wm, m));
  const int srows = __builtin_amdgcn_readfirstlane(min(m - srow0, 64));
  const __amdgpu_buffer_rsrc_t rs_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a_scale + int64_t(srow0) * groups), 0, srows * groups * 4,
      kBufferDword3);
  const int rs_off = lane * groups * 4;
  const int wrow =
      __builtin_amdgcn_readfirstlane(min((n0 + kWaveCols * wn) >> 7, (n >> 7) - 1));
  const float* __restrict__ wsp = w_scale + int64_t(wrow) * groups;
  // Copy block w + kWaves q of an operand is block w's offset plus 8 kWaves q rows; the sum
  // is formed at each copy from an opaque copy of block w's, so it costs one add, not a
  // live register.
  const int voff0 =
      (8 * wave + (lane >> 3)) * k + (((lane & 7) ^ (lane >> 3) ^ (wave & 1)) << 4);
  auto voff = [&](int q) {
    int v = voff0;
    asm volatile("" : "+v"(v));
    return v + q * 8 * kWaves * k;
  };

  // The copies of a step, in pieces: j < 4 the activation blocks of group ga, then its
  // row scales, then the kBBlocks weight blocks of group gb, then the weight scale of group
  // ga (a scalar load, issued where the step has no LDS read left to wait for: scalar and
  // LDS loads share a wait counter).  Past the last group the operand copies read a
  // zero-size buffer (zeros written, no memory traffic) and the scale loads repeat the last
  // group.  Every copy is unconditional: a branch here would split the step and let the
  // compiler sink its FMAs past the next barrier.
  constexpr int kPieces = kABlocks + 1 + kBBlocks + 1;
  auto copy_piece = [&](uint8_t* sa, uint8_t* sb, Scales& sc, int ga, int gb, int j) {
    if (j < kABlocks) {
      const bool live = ga < groups;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(live ? ra_rsrc : none_rsrc,
                                               (lds_void*)(sa + (wave + kWaves * j) * 1024),
                                               16, voff(j), live ? ga * 128 : 0, 0, 0);
    } else if (j == kABlocks) {
      sc.row = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(rs_rsrc, rs_off,
                                                      min(ga, groups - 1) * 4, 0));
    } else if (j < kABlocks + 1 + kBBlocks) {
      const int q = j - kABlocks - 1;
      const bool live = gb < groups;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(live ? rb_rsrc : none_rsrc,
                                               (lds_void*)(sb + (wave + kWaves * q) * 1024),
                                               16, voff(q), live ? gb * 128 : 0, 0, 0);
    } else {
      sc.w = wsp[min(ga, groups - 1)];
    }
  };

  v4f acc[4][kCols];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < kCols; ++c) acc[i][c] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  const Frag fo = frag_offsets(lane, wm, wn, kWaveCols);
  const int sel = (lane & 15) * 4;  // lane 16 i + orow holds row 16 i + orow's scale

  // Wait for this wave's copies of group g and its scales (everything but the previous
  // step's weight copies of group g + 1), then the barrier: everyone's copies of group g
  // landed and everyone is done reading the slots the next copies go to.  No fence: it
  // would drain the copies still in flight.  (vmcnt in bits 3:0 and 15:14, lgkmcnt 0,
  // expcnt not waited for.)
  constexpr int kWait = (kBBlocks & 15) | (7 << 4) | ((kBBlocks >> 4) << 14);
  using Deal = DealColumns<kCols, kABlocks, kPieces>;
  static_assert(Deal::valid(), "copy pieces dealt in index order, the scalar load last");
  auto barrier = [&]() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kWait);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  // Group g from slots (sa, sb) with scales sc; the activation copies and scales of group
  // g + 1 go to (na, nsc) and the weight copies of group g + 2 to nb, slots that held group
  // g - 1 (read by everyone before the barrier).  The copies are dealt out over the first
  // half of the step's MFMAs (deal_column) rather than issued in one burst ahead of them
  // (the burst queues in the address unit and holds back the MFMAs that follow it in the
  // wave's instruction stream).  Column 0 starts once B_0, A_0 and A_1 are in: each later
  // fragment is read one
  // MFMA ahead of its use; the column loop is software-pipelined (column c + 1's weight
  // fragment read and column c - 1's products scaled while column c multiplies, MFMA and
  // four FMAs alternating).
  auto step = [&](int g, const uint8_t* sa, const uint8_t* sb, const Scales& sc, uint8_t* na,
                  uint8_t* nb, Scales& nsc) {
    barrier();
    // Opaque copies of the fragment offsets: the addresses below are formed from them
    // within the step (one add per slot, the rest in the instruction's offset field)
    // instead of being hoisted out of the loop as one live register per slot and fragment.
    int alo = fo.a_lo, ahi = fo.a_hi, blo = fo.b_lo, bhi = fo.b_hi;
    asm volatile("" : "+v"(alo), "+v"(ahi), "+v"(blo), "+v"(bhi));
    copy_piece(na, nb, nsc, g + 1, g + 2, 0);
    v8i af[4];
    v4f pcur[4], pprev[4];
    v8i bcur = ld32(sb, blo, bhi);
    af[0] = ld32(sa, alo, ahi);
    af[1] = ld32(sa + 2048, alo, ahi);
    __builtin_amdgcn_sched_barrier(0);
    pcur[0] = mfma_group(bcur, af[0]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (Deal::column(1) == 0) copy_piece(na, nb, nsc, g + 1, g + 2, 1);
    __builtin_amdgcn_sched_barrier(0);
    af[2] = ld32(sa + 2 * 2048, alo, ahi);
    __builtin_amdgcn_sched_barrier(0);
    pcur[1] = mfma_group(bcur, af[1]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (Deal::column(2) == 0) copy_piece(na, nb, nsc, g + 1, g + 2, 2);
    __builtin_amdgcn_sched_barrier(0);
    af[3] = ld32(sa + 3 * 2048, alo, ahi);
    __builtin_amdgcn_sched_barrier(0);
    pcur[2] = mfma_group(bcur, af[2]);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (Deal::column(3) == 0) copy_piece(na, nb, nsc, g + 1, g + 2, 3);
    __builtin_amdgcn_sched_barrier(0);
    v8i bnxt = ld32(sb + 2048, blo, bhi);
    // the four row scales of this lane, times the weight scale (one product per row and
    // group, as the definition scales each group's partial)
    const int rsw = __builtin_bit_cast(int, sc.row * sc.w);
    int sel_here = sel;  // (opaque: one address register, the rest in the offset field)
    asm volatile("" : "+v"(sel_here));
    float f[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      f[i] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(sel_here + 64 * i, rsw));
    __builtin_amdgcn_sched_barrier(0);
    pcur[3] = mfma_group(bcur, af[3]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) pprev[i] = pcur[i];
    bcur = bnxt;
#pragma unroll
    for (int c = 1; c <= kCols; ++c) {
#pragma unroll
      for (int j = 1; j < kPieces; ++j)
        if (Deal::column(j) == c) copy_piece(na, nb, nsc, g + 1, g + 2, j);
      __builtin_amdgcn_sched_barrier(0);
      bnxt = bcur;
      if (c + 1 < kCols) bnxt = ld32(sb + (c + 1) * 2048, blo, bhi);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (c < kCols) pcur[i] = mfma_group(bcur, af[i]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][c - 1][j] = __builtin_fmaf(pprev[i][j], f[i], acc[i][c - 1][j]);
      }
      if (c < kCols) {  // MFMA, its neighbour's four FMAs, MFMA, ...
        if (c + 1 < kCols) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4; ++i) pprev[i] = pcur[i];
      bcur = bnxt;
    }
  };

  // Prologue: the activation copies and scales of group 0 and the weight copies of groups
  // 0 and 1, in issue order (the barrier's wait count assumes it, so no load may move).
  Scales s0, s1;
#pragma unroll
  for (int j = 0; j < kPieces; ++j) {
    copy_piece(st.x4, st.x0, s0, 0, 0, j);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int j = kABlocks + 1; j < kABlocks + 1 + kBBlocks; ++j) {
    copy_piece(st.x4, st.x1, s0, 0, 1, j);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  }
  int g = 0;
  do {  // (do-while: a guard before the first trip would let the prologue's loads sink)
    step(g, st.x4, st.x0, s0, st.x3, st.x2, s1);
    step(g + 1, st.x3, st.x1, s1, st.x4, st.x0, s0);
    step(g + 2, st.x4, st.x2, s0, st.x1, st.x3, s1);
    step(g + 3, st.x1, st.x0, s1, st.x4, st.x2, s0);
    step(g + 4, st.x4, st.x3, s0, st.x0, st.x1, s1);
    step(g + 5, st.x0, st.x2, s1, st.x4, st.x3, s0);
    step(g + 6, st.x4, st.x1, s0, st.x2, st.x0, s1);
    step(g + 7, st.x2, st.x3, s1, st.x4, st.x1, s0);
    g += 8;
  } while (g < groups);
  __syncthreads();  // every copy landed and every wave is done reading the slots
  store_tile<kWM, kWN, kCols>(acc, st.x0, st.x1, st.x2, st.x3, out, m, n, ldc, vec_out, m0,
                              n0);
}

}  // namespace ring

namespace tile256 {

constexpr int kBM = 256, kBN = 256, kThreads = 512;
constexpr int kArr = kBM * 128;           // one operand tile of one group (bytes)
constexpr int kGroupM = 4;                // row tiles per column tile in the walk order

// Work item -> output tile origin.  Items [0, n_full) are whole tiles, the rest the two
// halves (half 0 or 1: columns n0 .. n0 + 127) of each of the last tiles of the walk order;
// half is -1 for a whole tile.  The walk takes kGroupM consecutive row tiles per column
// tile, and each XCD (workgroup ids are dealt to the 8 XCDs round-robin) a contiguous
// stretch of it.
struct TileOrigin {
  int m0, n0, half;
};
__device__ __forceinline__ TileOrigin walk_tile(int item, int tiles_m, int tiles_n, int n_full) {
  int tile = item, half = -1;
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
  return {tm * kBM, tn * kBN + (half > 0 ? 128 : 0), half};
}

// Five-slot ring (group counts that are a multiple of eight): whole tiles 256 x 256, the
// halves 256 x 128, 32 KB slots (all 160 KB of LDS).
__global__ __launch_bounds__(kThreads, 1) void w8a8_prefill_ring_kernel(
    const uint8_t* __restrict__ a_q, const float* __restrict__ a_scale,
    const uint8_t* __restrict__ w_q, const float* __restrict__ w_scale,
    uint16_t* __restrict__ out, int m, int n, int k, int ldc, int tiles_m, int tiles_n,
    int n_full, int vec_out) {
  __shared__ __attribute__((aligned(16))) uint8_t x0[kArr], x1[kArr], x2[kArr], x3[kArr],
      x4[kArr];
  const ring::Slots<kArr> st{x0, x1, x2, x3, x4};
  const TileOrigin o = walk_tile(int(blockIdx.x), tiles_m, tiles_n, n_full);
  if (o.half < 0)
    ring::prefill_tile<4, 2, 8>(a_q, a_scale, w_q, w_scale, out, m, n, k, ldc, vec_out, o.m0,
                                o.n0, st);
  else
    ring::prefill_tile<4, 2, 4>(a_q, a_scale, w_q, w_scale, out, m, n, k, ldc, vec_out, o.m0,
                                o.n0, st);
}


// ---------------------------------------------------------------------------------------
// Two stages (any group count).
//
// Each stage holds one group's activation and weight tiles and its scales; group g
// multiplies from one while the copies of group g + 1 land in the other.  The operand
// arrays are separate objects: the compiler can then see that a stage's operand reads
// never alias the copies landing in the other stage, and keeps those copies in flight.
namespace two_stage {

struct Stages {
  uint8_t (&a0)[kArr];
  uint8_t (&a1)[kArr];
  uint8_t (&b0)[kArr];
  uint8_t (&b1)[kArr];
  float (&s0)[kBM + 32];
  float (&s1)[kBM + 32];
};

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
  // wave w fills copy blocks w + 8q of each operand
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

  // The copies of group g, in pieces: j < 4 the activation blocks, then the kBBlocks weight
  // blocks, then the scales.  Outside [0, groups) they read a zero-size buffer (zeros
  // written, no memory traffic) and repeat a valid scale.  Every copy is unconditional: a
  // branch here would split the step and let the compiler sink its FMAs past the next
  // barrier.
  constexpr int kPieces = 4 + kBBlocks + 1;
  auto copy_piece = [&](uint8_t* sa, uint8_t* sb, float* ss, int g, int j) {
    const bool live = g >= 0 && g < groups;
    const int goff = live ? g * 128 : 0;
    if (j < 4)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(live ? ra_rsrc : none_rsrc,
                                               (lds_void*)(sa + (wave + 8 * j) * 1024), 16,
                                               voff[j], goff, 0, 0);
    else if (j < 4 + kBBlocks)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(live ? rb_rsrc : none_rsrc,
                                               (lds_void*)(sb + (wave + 8 * (j - 4)) * 1024),
                                               16, voff[j - 4], goff, 0, 0);
    else
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(gsp + min(max(g, 0), groups - 1)),
          (lds_void*)(ss + 32 * wave), 4, 0, 0);
  };

  v4f acc[4][kCols];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < kCols; ++c) acc[i][c] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  const Frag fo = frag_offsets(lane, wm, wn, kWaveCols);
  const int s_off = (wm * 64 + (lane & 15)) * 4;  // row 64 wm + orow's scale slot

  // Group g from stage (sa, sb, ss); the copies of group g + 1 go to (na, nbs, ns), which
  // held group g - 1 (read by everyone before the barrier).  The copies are dealt out over
  // the first half of the step's MFMAs, one piece after each.
  auto step = [&](int g, const uint8_t* sa, const uint8_t* sb, const float* ss, uint8_t* na,
                  uint8_t* nbs, float* ns) {
    __syncthreads();  // everyone's copies of group g landed (the fence drains them)
    copy_piece(na, nbs, ns, g + 1, 0);
    v8i af[4];
    float as[4];
    v4f pcur[4], pprev[4];
    v8i bcur = ld32(sb, fo.b_lo, fo.b_hi);
    af[0] = ld32(sa, fo.a_lo, fo.a_hi);
    af[1] = ld32(sa + 2048, fo.a_lo, fo.a_hi);
    __builtin_amdgcn_sched_barrier(0);
    pcur[0] = mfma_group(bcur, af[0]);
    __builtin_amdgcn_sched_barrier(0);
    copy_piece(na, nbs, ns, g + 1, 1);
    __builtin_amdgcn_sched_barrier(0);
    af[2] = ld32(sa + 2 * 2048, fo.a_lo, fo.a_hi);
    __builtin_amdgcn_sched_barrier(0);
    pcur[1] = mfma_group(bcur, af[1]);
    __builtin_amdgcn_sched_barrier(0);
    copy_piece(na, nbs, ns, g + 1, 2);
    __builtin_amdgcn_sched_barrier(0);
    af[3] = ld32(sa + 3 * 2048, fo.a_lo, fo.a_hi);
    __builtin_amdgcn_sched_barrier(0);
    pcur[2] = mfma_group(bcur, af[2]);
    __builtin_amdgcn_sched_barrier(0);
    copy_piece(na, nbs, ns, g + 1, 3);
    __builtin_amdgcn_sched_barrier(0);
    v8i bnxt = ld32(sb + 2048, fo.b_lo, fo.b_hi);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      as[i] = *reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(ss) + s_off +
                                              i * 64);
    const float ws = ss[kBM + wn];
    __builtin_amdgcn_sched_barrier(0);
    pcur[3] = mfma_group(bcur, af[3]);
    __builtin_amdgcn_sched_barrier(0);
    float f[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = as[i] * ws;
      pprev[i] = pcur[i];
    }
    bcur = bnxt;
#pragma unroll
    for (int c = 1; c <= kCols; ++c) {
      if (3 + c < kPieces) copy_piece(na, nbs, ns, g + 1, 3 + c);
      __builtin_amdgcn_sched_barrier(0);
      bnxt = bcur;
      if (c + 1 < kCols) bnxt = ld32(sb + (c + 1) * 2048, fo.b_lo, fo.b_hi);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (c < kCols) pcur[i] = mfma_group(bcur, af[i]);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][c - 1][j] = __builtin_fmaf(pprev[i][j], f[i], acc[i][c - 1][j]);
      }
      if (c < kCols) {  // MFMA, its neighbour's four FMAs, MFMA, ...
        if (c + 1 < kCols) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
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
#pragma unroll
  for (int j = 0; j < kPieces; ++j) copy_piece(st.a0, st.b0, st.s0, -odd, j);
  for (int g = -odd; g < groups; g += 2) {
    step(g, st.a0, st.b0, st.s0, st.a1, st.b1, st.s1);
    step(g + 1, st.a1, st.b1, st.s1, st.a0, st.b0, st.s0);
  }
  __syncthreads();  // every copy landed and every wave is done reading the stages
  store_tile<4, 2, kCols>(acc, st.a0, st.a1, st.b0, st.b1, out, m, n, ldc, vec_out, m0, n0);
}

__global__ __launch_bounds__(kThreads, 1) void w8a8_prefill_kernel(
    const uint8_t* __restrict__ a_q, const float* __restrict__ a_scale,
    const uint8_t* __restrict__ w_q, const float* __restrict__ w_scale,
    uint16_t* __restrict__ out, int m, int n, int k, int ldc, int tiles_m, int tiles_n,
    int n_full, int vec_out) {
  __shared__ __attribute__((aligned(16))) uint8_t a0[kArr], a1[kArr], b0[kArr], b1[kArr];
  __shared__ __attribute__((aligned(16))) float s0[kBM + 32], s1[kBM + 32];
  const Stages st{a0, a1, b0, b1, s0, s1};
  const TileOrigin o = walk_tile(int(blockIdx.x), tiles_m, tiles_n, n_full);
  if (o.half < 0)
    prefill_tile<8>(a_q, a_scale, w_q, w_scale, out, m, n, k, ldc, vec_out, o.m0, o.n0, st);
  else
    prefill_tile<4>(a_q, a_scale, w_q, w_scale, out, m, n, k, ldc, vec_out, o.m0, o.n0, st);
}

}  // namespace two_stage

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

// Workgroup -> output tile origin (m0, n0): kGroupM consecutive row tiles per column tile,
// each XCD a contiguous stretch of that order.
__device__ __forceinline__ int2 tile_origin(int bid, int tiles_m, int tiles_n) {
  const int nblk = tiles_m * tiles_n;
  const int even = nblk - nblk % kXcds;
  if (bid < even) bid = (bid % kXcds) * (even / kXcds) + bid / kXcds;
  const int band = kGroupM * tiles_n;
  const int first_m = (bid / band) * kGroupM;
  const int band_m = min(kGroupM, tiles_m - first_m);
  const int tm = first_m + (bid % band) % band_m;
  const int tn = (bid % band) / band_m;
  return make_int2(tm * kBM, tn * kBN);
}

// Five-slot ring (group counts that are a multiple of eight, at most one tile per CU):
// 16 KB slots, 2 x 2 waves of 64 x 64.
constexpr int kRingWN = 2, kRingCols = 4;
constexpr int kRingThreads = 128 * kRingWN;
__global__ __launch_bounds__(kRingThreads, 2) void w8a8_prefill_small_ring_kernel(
    const uint8_t* __restrict__ a_q, const float* __restrict__ a_scale,
    const uint8_t* __restrict__ w_q, const float* __restrict__ w_scale,
    uint16_t* __restrict__ out, int m, int n, int k, int ldc, int tiles_m, int tiles_n,
    int vec_out) {
  static_assert(kAStage == kBStage, "one slot size for both operands");
  __shared__ __attribute__((aligned(16))) uint8_t x0[kAStage], x1[kAStage], x2[kAStage],
      x3[kAStage], x4[kAStage];
  const ring::Slots<kAStage> st{x0, x1, x2, x3, x4};
  const int2 origin = tile_origin(int(blockIdx.x), tiles_m, tiles_n);
  ring::prefill_tile<2, kRingWN, kRingCols>(a_q, a_scale, w_q, w_scale, out, m, n, k, ldc,
                                            vec_out, origin.x, origin.y, st);
}

// Two stages (any group count).
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

  const int2 origin = tile_origin(int(blockIdx.x), tiles_m, tiles_n);
  const int m0 = origin.x, n0 = origin.y;

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
    // the five-slot ring's rotation repeats every eight groups
    const auto kernel = (k / 128) % 8 == 0 ? tile256::w8a8_prefill_ring_kernel
                                            : tile256::two_stage::w8a8_prefill_kernel;
    launch(kernel, dim3(unsigned(n_full + 2 * split)), dim3(tile256::kThreads), 0, stream, a_q,
           a_scale, w_q, w_scale, out, m, n, k, ldc, int(big_m), int(big_n), int(n_full),
           vec_out);
    return launch_status();
  }
  const int64_t tiles_m = (int64_t(m) + 127) / 128, tiles_n = (int64_t(n) + 127) / 128;
  if (tiles_m * tiles_n > 0x7FFFFFFF) return FP8Q_EINVAL;
  // the ring when every CU holds at most one tile (with two tiles side by side on a CU its
  // deeper copies gain nothing)
  const bool ring = (k / 128) % 8 == 0 && tiles_m * tiles_n <= cus;
  launch(ring ? tile128::w8a8_prefill_small_ring_kernel : tile128::w8a8_prefill_small_kernel,
         dim3(unsigned(tiles_m * tiles_n)),
         dim3(ring ? tile128::kRingThreads : tile128::kThreads), 0, stream, a_q, a_scale, w_q,
         w_scale, out, m, n, k, ldc, int(tiles_m), int(tiles_n), vec_out);
  return launch_status();
}
