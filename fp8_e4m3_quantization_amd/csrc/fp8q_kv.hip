// fp8q_kv.hip -- paged FP8 KV-cache write at a per-tensor scale, the K/V absolute
// maximum that feeds the online calibration, and the dequantizing read of a history.
//
// staging.rs page: Fp8KvWriteTarget (strides in elements, pool stride = block_size *
// heads * head_dim per block) and replay_and_release (the write's argument list); module
// doc (one scale per tensor; chronological rewrites, last writer wins).
// fp8_calibration.rs page: Fp8KvCalibration::absmax (max |K| and max |V|,
// max-accumulated into a zeroed float pair).
//
// Layout inside a block is [offset][head][dim] (the pages give only the per-block stride
// block_size*H*D, which this reading fills exactly), so one token's H*D codes are
// contiguous: the write is a gather-free row copy-convert into a slot-addressed row.
// Vector path: a thread converts 8 elements of K and the same 8 of V (two 16-byte loads,
// two 8-byte stores); with H*D = 512 a wave covers one token, so the slot load is a
// broadcast.  Division by the scale is the remainder-corrected reciprocal product with
// an estimate clip (any positive scale is accepted; out-of-range values saturate).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8q.h"
#include "fp8q_device.h"
#include "fp8q_kv_internal.h"
#include "fp8q_launch.h"

#pragma clang fp contract(off)

namespace fp8q {
namespace {

constexpr int kKvBlock = 256;
// Threads per block of the wide write: one pass over the tokens in 512-thread blocks.
// Measured against 256 and 1024 threads and against persistent grids of 2 to 8 blocks per
// CU with one to four tokens' loads in flight per wave: none was faster.
constexpr int kWideBlock = 512;

__device__ __forceinline__ bool slot_to_block(int64_t slot, int64_t nslots, int bs,
                                              int64_t* blk, int64_t* off) {
  if (slot < 0 || slot >= nslots) return false;
  if (nslots <= 0x7FFFFFFF) {
    const uint32_t s = uint32_t(slot);
    *blk = int64_t(s / uint32_t(bs));
    *off = int64_t(s % uint32_t(bs));
  } else {
    *blk = slot / bs;
    *off = slot % bs;
  }
  return true;
}

// Thread layout for every kernel below: blockDim = (64, 4), one wave per token row, so
// a row's slot is uniform across the wave and read once into a scalar register.
constexpr int kRowsPerBlock = 4;

__device__ __forceinline__ int64_t uniform(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(v)));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(v) >> 32));
  return int64_t((uint64_t(hi) << 32) | lo);
}

// ept = elements per token / 8; ks8, vs8 = source row strides / 8; cs8 = pool stride / 8.
// A wave takes kTokPerWave consecutive tokens: their slots are read first (scalar loads),
// then every 16-byte load of the group is issued before any conversion, so each wave
// keeps 2 * kTokPerWave loads in flight instead of waiting on one token at a time.
constexpr int kTokPerWave = 4;

__global__ __launch_bounds__(kKvBlock) void kv_write_vec_kernel(
    const uint4* __restrict__ k, const uint4* __restrict__ v, uint2* __restrict__ kc,
    uint2* __restrict__ vc, const int64_t* __restrict__ slots, int64_t num_tokens, int ept,
    int64_t ks8, int64_t vs8, int64_t cs8, int bs, int64_t nslots, float k_scale,
    float k_inv, float v_scale, float v_inv) {
  const int64_t step = int64_t(gridDim.x) * kRowsPerBlock * kTokPerWave;
  for (int64_t t0 = (int64_t(blockIdx.x) * kRowsPerBlock + threadIdx.y) * kTokPerWave;
       t0 < num_tokens; t0 += step) {
    int64_t tok[kTokPerWave], dst[kTokPerWave];
    bool ok[kTokPerWave];
#pragma unroll
    for (int i = 0; i < kTokPerWave; ++i) {
      const int64_t t = t0 + i;
      tok[i] = t < num_tokens ? t : num_tokens - 1;  // clamped: loads stay in bounds
      int64_t blk = 0, off = 0;
      ok[i] = t < num_tokens && slot_to_block(uniform(slots[tok[i]]), nslots, bs, &blk, &off);
      dst[i] = blk * cs8 + off * ept;
    }
    for (int c = threadIdx.x; c < ept; c += 64) {
      uint4 kx[kTokPerWave], vx[kTokPerWave];
#pragma unroll
      for (int i = 0; i < kTokPerWave; ++i) {
        kx[i] = k[tok[i] * ks8 + c];
        vx[i] = v[tok[i] * vs8 + c];
      }
#pragma unroll
      for (int i = 0; i < kTokPerWave; ++i) {
        if (ok[i]) {
          const uint2 kq = quant8<false>(kx[i], k_scale, k_inv);
          const uint2 vq = quant8<false>(vx[i], v_scale, v_inv);
          __builtin_nontemporal_store(uint64_t(kq.x) | (uint64_t(kq.y) << 32),
                                      reinterpret_cast<uint64_t*>(kc + dst[i] + c));
          __builtin_nontemporal_store(uint64_t(vq.x) | (uint64_t(vq.y) << 32),
                                      reinterpret_cast<uint64_t*>(vc + dst[i] + c));
        }
      }
    }
  }
}

// Wide form for rows of e = 16 * lpt elements with 2 * lpt dividing 64 (e = 16 .. 512):
// a token takes 2 * lpt lanes -- the first lpt convert 16 elements of its K row each (two
// 16-byte loads, one 16-byte store), the next lpt the same 16 elements of its V row -- so a
// wave covers 64 / (2 * lpt) tokens per step and every store instruction writes whole
// 16-byte lanes.

// Codes of a lane's 16 elements: one 16-byte store with the non-temporal hint (the pool is
// not read again by this kernel), so each store instruction writes whole lines.
__device__ __forceinline__ void store16_nt(uint4 v, uint8_t* p) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(v4u{v.x, v.y, v.z, v.w}, reinterpret_cast<v4u*>(p));
}

// The value of amax2[which] as the kernel starts, read by the thread that later folds into
// it.  The slot only grows, so this early read is never larger than the slot's value at
// fold time: skipping the atomic when the block's maximum does not exceed it stays
// correct, and the read's latency hides under the kernel's own loads.
__device__ __forceinline__ float seen_max(float* amax2, int which) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<unsigned int*>(amax2 + which),
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// Folds a workgroup's two maxima (K, V) into amax2[0..1]: wave DPP max, one LDS round, one
// atomic each (skipped when `seen`, thread t's seen_max(amax2, t), is already as large).
template <int kBlock>
__device__ __forceinline__ void fold_block_max2(float mk, float mv, float* amax2, float seen) {
  __shared__ float red[2][kBlock / 64];
  const int tid = threadIdx.x;
  mk = max_over_wave(mk);
  mv = max_over_wave(mv);
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = mk;
    red[1][tid >> 6] = mv;
  }
  __syncthreads();
  if (tid < 2) {
    float b = red[tid][0];
    for (int w = 1; w < kBlock / 64; ++w) b = fmaxf(b, red[tid][w]);
    if (b > 0.0f && __float_as_uint(b) > __float_as_uint(seen))
      atomicMax(reinterpret_cast<unsigned int*>(amax2 + tid), __float_as_uint(b));
  }
}

// lpt = 1 << lpt_log2 (2 * lpt divides 64, so lpt is a power of two: lane arithmetic is
// shifts and masks).  kAmax: also max-accumulate max|K| and max|V| of every row
// t < num_tokens (whatever its slot) into amax2, from the same loads.
template <bool kAmax>
__global__ __launch_bounds__(kWideBlock) void kv_write_wide_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, uint8_t* __restrict__ kc,
    uint8_t* __restrict__ vc, const int64_t* __restrict__ slots, int64_t num_tokens,
    int lpt_log2, int64_t ks, int64_t vs, int64_t cs, int bs, int64_t nslots, float k_scale,
    float k_inv, float v_scale, float v_inv, float* __restrict__ amax2) {
  const int lane = threadIdx.x & 63;
  const int lpt = 1 << lpt_log2;
  const int tpw = 64 >> (lpt_log2 + 1);             // tokens per wave per step
  const int slot_in_wave = lane >> (lpt_log2 + 1);  // which of those tokens
  const int half = (lane >> lpt_log2) & 1;          // 0: K, 1: V
  const int chunk = lane & (lpt - 1);               // 16-element chunk within the row
  const int e = 16 * lpt;
  const uint16_t* src = half ? v : k;
  const int64_t sstride = half ? vs : ks;
  uint8_t* dpool = half ? vc : kc;
  const float sc = half ? v_scale : k_scale, inv = half ? v_inv : k_inv;
  const int64_t wave = (int64_t(blockIdx.x) * kWideBlock + threadIdx.x) >> 6;
  const int64_t nwaves = (int64_t(gridDim.x) * kWideBlock) >> 6;
  float mx = 0.0f;  // kAmax: this lane's running max |x|
  const float seen = (kAmax && threadIdx.x < 2) ? seen_max(amax2, int(threadIdx.x)) : 0.0f;
  for (int64_t t0 = wave * tpw; t0 < num_tokens; t0 += nwaves * tpw) {
    const int64_t tok = t0 + slot_in_wave;
    const int64_t tl = tok < num_tokens ? tok : num_tokens - 1;  // in bounds
    const uint4* p = reinterpret_cast<const uint4*>(src + tl * sstride + chunk * 16);
    const uint4 x0 = p[0], x1 = p[1];
    int64_t blk = 0, off = 0;
    const bool ok = tok < num_tokens && slot_to_block(slots[tl], nslots, bs, &blk, &off);
    const uint2 a = quant8<false>(x0, sc, inv);
    const uint2 b = quant8<false>(x1, sc, inv);
    if (ok) store16_nt(make_uint4(a.x, a.y, b.x, b.y), dpool + blk * cs + off * e + chunk * 16);
    if (kAmax && tok < num_tokens) mx = fmaxf(mx, fmaxf(absmax8(x0), absmax8(x1)));
  }
  if constexpr (kAmax) fold_block_max2<kWideBlock>(half ? 0.0f : mx, half ? mx : 0.0f, amax2, seen);
}

__device__ __forceinline__ uint8_t e4m3_one(float v) {
  return uint8_t(__builtin_amdgcn_cvt_pk_fp8_f32(clip448(v), 0.0f, 0, false) & 0xFF);
}

// Element-wise path for any geometry and alignment.
__global__ __launch_bounds__(kKvBlock) void kv_write_scalar_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, uint8_t* __restrict__ kc,
    uint8_t* __restrict__ vc, const int64_t* __restrict__ slots, int64_t num_tokens, int e,
    int64_t ks, int64_t vs, int64_t cs, int bs, int64_t nslots, float k_scale, float k_inv,
    float v_scale, float v_inv) {
  for (int64_t t = int64_t(blockIdx.x) * kRowsPerBlock + threadIdx.y; t < num_tokens;
       t += int64_t(gridDim.x) * kRowsPerBlock) {
    int64_t blk, off;
    if (!slot_to_block(uniform(slots[t]), nslots, bs, &blk, &off)) continue;
    const int64_t dst = blk * cs + off * e;
    for (int c = threadIdx.x; c < e; c += 64) {
      kc[dst + c] = e4m3_one(div_by_scale_clipped(bf16_to_f32(k[t * ks + c]), k_scale, k_inv));
      vc[dst + c] = e4m3_one(div_by_scale_clipped(bf16_to_f32(v[t * vs + c]), v_scale, v_inv));
    }
  }
}

// ------------------------------------------------------------------ dequantizing read
// Gather of a paged history back to bf16 at one scale per tensor: every element is
// bf16_rne(fp32(decode(code)) * scale).  Work item = the same 8 elements of one token's K
// and V rows: item i -> token i / ipt (ipt = H*D/8 items per token), chunk i % ipt.  A lane
// loads 8 K codes and 8 V codes and stores 16 bf16 bytes of each output row; consecutive
// lanes take consecutive chunks, so every load instruction of a wave reads 512 contiguous
// bytes of a pool row and every store writes 1 KB of an output row in whole 16-byte lanes
// (no instruction leaves holes in a cache line).  A lane takes kReadUnroll items a pass,
// all loads issued before any conversion.  Tokens whose slot is out of range read pool
// row 0 (in bounds) and store nothing.
// A lane takes four items a pass (all loads issued before any conversion), in 256-thread
// blocks, and writes its bf16 rows with the non-temporal hint; measured against 128/512
// threads and other unrolls.
constexpr int kReadUnroll = 4;
constexpr int kReadBlock = 256;  // threads per block of the vector read

__device__ __forceinline__ void store16_bf16(uint4 a, uint16_t* p) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  __builtin_nontemporal_store(v4u{a.x, a.y, a.z, a.w}, reinterpret_cast<v4u*>(p));
}

__device__ __forceinline__ uint4 dequant8(uint2 w, float s) {
  const uint2 a = dequant4(w.x, s), b = dequant4(w.y, s);
  return make_uint4(a.x, a.y, b.x, b.y);
}

__device__ __forceinline__ uint4 dequant8_finite(uint2 w, float s) {
  const uint2 a = dequant4_finite(w.x, s), b = dequant4_finite(w.y, s);
  return make_uint4(a.x, a.y, b.x, b.y);
}

// Idx is uint32_t when every item index and slot fits in 31 bits, else uint64_t; kPow2:
// ipt is a power of two (ipt_log2 its exponent), so token and chunk are a shift and a mask.
template <typename Idx, bool kPow2>
__global__ __launch_bounds__(kReadBlock) void kv_read_vec_kernel(
    const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
    const int64_t* __restrict__ slots, Idx items, uint32_t ipt, uint32_t ipt_log2, int64_t cs,
    uint32_t bs, int64_t nslots, float k_scale, float v_scale, uint16_t* __restrict__ ko,
    uint16_t* __restrict__ vo, int64_t kos, int64_t vos) {
  const Idx nthreads = Idx(gridDim.x) * kReadBlock;
  const int64_t e = int64_t(8) * ipt;
  for (Idx i0 = Idx(blockIdx.x) * kReadBlock + threadIdx.x; i0 < items;
       i0 += nthreads * kReadUnroll) {
    Idx tok[kReadUnroll], c[kReadUnroll];
    int64_t slot[kReadUnroll];
    // every slot load first (clamped items: in bounds), then every pool load
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const Idx i = i0 + u * nthreads;
      const Idx il = i < items ? i : items - 1;
      tok[u] = kPow2 ? il >> ipt_log2 : il / ipt;
      c[u] = il - tok[u] * ipt;
      slot[u] = slots[tok[u]];
    }
    uint2 kw[kReadUnroll], vw[kReadUnroll];
    bool ok[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      ok[u] = i0 + u * nthreads < items && slot[u] >= 0 && slot[u] < nslots;
      const Idx su = ok[u] ? Idx(slot[u]) : Idx(0);  // invalid: row 0 of block 0
      const Idx blk = su / bs;
      const Idx off = su - blk * bs;
      const int64_t src = int64_t(blk) * cs + int64_t(off) * e + int64_t(c[u]) * 8;
      kw[u] = *reinterpret_cast<const uint2*>(kc + src);
      vw[u] = *reinterpret_cast<const uint2*>(vc + src);
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      // hardware bf16 conversion unless a NaN code is present (then the exact integer path)
      const uint32_t nan = e4m3_nan_bytes(kw[u].x) | e4m3_nan_bytes(kw[u].y) |
                           e4m3_nan_bytes(vw[u].x) | e4m3_nan_bytes(vw[u].y);
      uint4 kd, vd;
      if (__builtin_expect(nan == 0, 1)) {
        kd = dequant8_finite(kw[u], k_scale);
        vd = dequant8_finite(vw[u], v_scale);
      } else {
        kd = dequant8(kw[u], k_scale);
        vd = dequant8(vw[u], v_scale);
      }
      if (ok[u]) {
        store16_bf16(kd, ko + int64_t(tok[u]) * kos + int64_t(c[u]) * 8);
        store16_bf16(vd, vo + int64_t(tok[u]) * vos + int64_t(c[u]) * 8);
      }
    }
  }
}

// Element-wise read for any geometry and alignment; one wave per token row.
__global__ __launch_bounds__(kKvBlock) void kv_read_scalar_kernel(
    const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
    const int64_t* __restrict__ slots, int64_t num_tokens, int e, int64_t cs, int bs,
    int64_t nslots, float k_scale, float v_scale, uint16_t* __restrict__ ko,
    uint16_t* __restrict__ vo, int64_t kos, int64_t vos) {
  for (int64_t t = int64_t(blockIdx.x) * kRowsPerBlock + threadIdx.y; t < num_tokens;
       t += int64_t(gridDim.x) * kRowsPerBlock) {
    int64_t blk, off;
    if (!slot_to_block(uniform(slots[t]), nslots, bs, &blk, &off)) continue;
    const int64_t src = blk * cs + off * e;
    for (int c = threadIdx.x; c < e; c += 64) {
      const float kd = e4m3x2_to_f32<false>(kc[src + c]).x;
      const float vd = e4m3x2_to_f32<false>(vc[src + c]).x;
      ko[t * kos + c] = uint16_t(f32_to_bf16_bits(kd * k_scale));
      vo[t * vos + c] = uint16_t(f32_to_bf16_bits(vd * v_scale));
    }
  }
}

// ------------------------------------------------------------ last-writer replay mask
// out[i] = -1 for every token i that a later token j > i of the same list writes over
// (same slot); out must already hold a copy of slots.  Block (bi, bj) is one wave that
// compares the 64 tokens of tile bi against the 64 of tile bj >= bi; every pair (i, j > i)
// is seen by exactly one block.  Blocks only store -1 into out and never read it, so their
// order does not matter.
__global__ __launch_bounds__(64) void kv_mark_superseded_kernel(
    const int64_t* __restrict__ slots, int64_t* __restrict__ out, int n) {
  const int bi = blockIdx.x, bj = blockIdx.y;
  if (bj < bi) return;
  const int i = bi * 64 + int(threadIdx.x);
  const int64_t si = slots[i < n ? i : n - 1];
  const int j0 = bj * 64;
  const int jn = n - j0 < 64 ? n - j0 : 64;
  bool superseded = false;
  for (int jj = 0; jj < jn; ++jj) superseded |= (j0 + jj > i) && (slots[j0 + jj] == si);
  if (i < n && superseded) out[i] = -1;
}

// Folds a workgroup's maximum into amax2[which]: one LDS reduction, then a single atomic,
// skipped when the value already there is at least as large (it only grows).
// seen: seen_max(amax2, which) as read by thread 0 at kernel start.
template <int kBlock>
__device__ __forceinline__ void fold_block_max(float m, float* amax2, int which, float seen) {
  __shared__ float red[kBlock / 64];
  const int tid = threadIdx.x + threadIdx.y * blockDim.x;
  m = max_over_wave(m);
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) {
    float b = red[0];
    for (int w = 1; w < kBlock / 64; ++w) b = fmaxf(b, red[w]);
    if (b > 0.0f && __float_as_uint(b) > __float_as_uint(seen))
      atomicMax(reinterpret_cast<unsigned int*>(amax2 + which), __float_as_uint(b));
  }
}

// max |x| over a packed run of n8 16-byte words; blockIdx.y picks K (0) or V (1).  Four
// independent 16-byte loads per thread per step keep enough bytes in flight; the loads carry
// the non-temporal hint (read once: measured 3-4 % faster than plain loads on the whole pool,
// where 256- and 512-thread blocks and persistent grids were slower).
constexpr int kAmaxBlock = 1024;
constexpr int64_t kAmaxMaxBlocks = 4096;  // per tensor
__global__ __launch_bounds__(kAmaxBlock) void amax_flat_kernel(const uint4* __restrict__ k,
                                                             const uint4* __restrict__ v,
                                                             int64_t n8,
                                                             float* __restrict__ amax2) {
  const uint4* x = blockIdx.y ? v : k;
  const float seen = threadIdx.x == 0 ? seen_max(amax2, int(blockIdx.y)) : 0.0f;
  const int64_t stride = int64_t(gridDim.x) * kAmaxBlock;
  float m = 0.0f;
  int64_t i = int64_t(blockIdx.x) * kAmaxBlock + threadIdx.x;
  typedef unsigned v4u_nt __attribute__((ext_vector_type(4)));
  const v4u_nt* xv = reinterpret_cast<const v4u_nt*>(x);
  auto ld = [&](int64_t j) {
    const v4u_nt t = __builtin_nontemporal_load(xv + j);
    return make_uint4(t[0], t[1], t[2], t[3]);
  };
  for (; i + 3 * stride < n8; i += 4 * stride) {
    const uint4 a = ld(i), b = ld(i + stride), c = ld(i + 2 * stride), d = ld(i + 3 * stride);
    m = fmaxf(m, fmaxf(fmaxf(absmax8(a), absmax8(b)), fmaxf(absmax8(c), absmax8(d))));
  }
  for (; i < n8; i += stride) m = fmaxf(m, absmax8(ld(i)));
  fold_block_max<kAmaxBlock>(m, amax2, blockIdx.y, seen);
}

// max |x| over `rows` rows of `row_elems` bf16 at row strides ks / vs (any alignment).
__global__ __launch_bounds__(kKvBlock) void amax_rows_kernel(const uint16_t* __restrict__ k,
                                                             const uint16_t* __restrict__ v,
                                                             int64_t rows, int row_elems,
                                                             int64_t ks, int64_t vs,
                                                             float* __restrict__ amax2) {
  const uint16_t* x = blockIdx.y ? v : k;
  const int64_t s = blockIdx.y ? vs : ks;
  const float seen = (threadIdx.x == 0 && threadIdx.y == 0) ? seen_max(amax2, int(blockIdx.y)) : 0.0f;
  float m = 0.0f;
  for (int64_t r = int64_t(blockIdx.x) * kRowsPerBlock + threadIdx.y; r < rows;
       r += int64_t(gridDim.x) * kRowsPerBlock)
    for (int c = threadIdx.x; c < row_elems; c += 64)
      m = fmaxf(m, fabsf(bf16_to_f32(x[r * s + c])));
  fold_block_max<kKvBlock>(m, amax2, blockIdx.y, seen);
}

// Staging of a calibration batch in one pass: `rows` rows of e = 8 * ce bf16 at strides
// ks / vs (elements) are copied packed to dk / dv (row t at t * e), their |K| / |V| maxima
// folded into amax2 (as amax_rows_kernel would), and the batch's int64 slots copied to
// dslots.  Work item = the same 16-byte chunk of one row of K and of V: item i -> row i / ce,
// chunk i % ce, so consecutive lanes read and write contiguous bytes.
constexpr int kStageBlock = 256;
__global__ __launch_bounds__(kStageBlock) void kv_stage_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int64_t* __restrict__ slots, int64_t rows, int64_t ce, int64_t ks, int64_t vs,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int64_t* __restrict__ dslots,
    float* __restrict__ amax2) {
  const float seen = threadIdx.x < 2 ? seen_max(amax2, int(threadIdx.x)) : 0.0f;
  const int64_t items = rows * ce;
  const int64_t stride = int64_t(gridDim.x) * kStageBlock;
  const int64_t first = int64_t(blockIdx.x) * kStageBlock + threadIdx.x;
  float mk = 0.0f, mv = 0.0f;
  for (int64_t i = first; i < items; i += stride) {
    const int64_t t = i / ce, c = i - t * ce;
    const uint4 a = *reinterpret_cast<const uint4*>(k + t * ks + c * 8);
    const uint4 b = *reinterpret_cast<const uint4*>(v + t * vs + c * 8);
    *reinterpret_cast<uint4*>(dk + i * 8) = a;
    *reinterpret_cast<uint4*>(dv + i * 8) = b;
    mk = fmaxf(mk, absmax8(a));
    mv = fmaxf(mv, absmax8(b));
  }
  for (int64_t i = first; i < rows; i += stride) dslots[i] = slots[i];
  fold_block_max2<kStageBlock>(mk, mv, amax2, seen);
}

}  // namespace

int kv_stage(const uint16_t* k, const uint16_t* v, const int64_t* slots, int64_t rows,
             int64_t e, int64_t key_stride, int64_t value_stride, uint16_t* dk, uint16_t* dv,
             int64_t* dslots, float* amax2, hipStream_t stream) {
  if (rows <= 0) return FP8Q_OK;
  const bool vec = e % 8 == 0 && key_stride % 8 == 0 && value_stride % 8 == 0 &&
                   aligned(k, 16) && aligned(v, 16) && aligned(dk, 16) && aligned(dv, 16) &&
                   aligned(slots, 8) && aligned(dslots, 8);
  if (vec) {
    const int64_t items = rows * (e / 8);
    int64_t blocks = (items + kStageBlock - 1) / kStageBlock;
    if (blocks > 1024) blocks = 1024;
    launch(kv_stage_kernel, dim3(unsigned(blocks)), dim3(kStageBlock), 0, stream, k, v, slots,
           rows, e / 8, key_stride, value_stride, dk, dv, dslots, amax2);
    return launch_status();
  }
  // other geometries: the absmax pass, then the row and slot copies
  int rc = kv_amax_rows(k, v, rows, e, key_stride, value_stride, amax2, stream);
  if (rc != FP8Q_OK) return rc;
  const size_t row = size_t(e) * 2;
  if (hipMemcpy2DAsync(dk, row, k, size_t(key_stride) * 2, row, size_t(rows),
                       hipMemcpyDeviceToDevice, stream) != hipSuccess ||
      hipMemcpy2DAsync(dv, row, v, size_t(value_stride) * 2, row, size_t(rows),
                       hipMemcpyDeviceToDevice, stream) != hipSuccess ||
      hipMemcpyAsync(dslots, slots, size_t(rows) * 8, hipMemcpyDeviceToDevice, stream) !=
          hipSuccess)
    return FP8Q_EHIP;
  return FP8Q_OK;
}

int kv_amax_rows(const uint16_t* k, const uint16_t* v, int64_t rows, int64_t row_elems,
                 int64_t key_stride, int64_t value_stride, float* amax2, hipStream_t stream) {
  if (rows == 0 || row_elems == 0) return FP8Q_OK;
  const int64_t n = rows * row_elems;
  if (key_stride == row_elems && value_stride == row_elems && n % 8 == 0 && aligned(k, 16) &&
      aligned(v, 16)) {
    // four 16-byte words per thread per step; enough blocks to fill every CU
    int64_t blocks = (n / 8 + 4 * kAmaxBlock - 1) / (4 * kAmaxBlock);
    if (blocks > kAmaxMaxBlocks) blocks = kAmaxMaxBlocks;
    launch(amax_flat_kernel, dim3(unsigned(blocks), 2), dim3(kAmaxBlock), 0, stream,
                       reinterpret_cast<const uint4*>(k), reinterpret_cast<const uint4*>(v),
                       n / 8, amax2);
  } else {
    if (row_elems > 0x7FFFFFFF) return FP8Q_EINVAL;
    int64_t blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
    if (blocks > 1024) blocks = 1024;
    launch(amax_rows_kernel, dim3(unsigned(blocks), 2), dim3(64, kRowsPerBlock), 0,
                       stream, k, v, rows, int(row_elems), key_stride, value_stride, amax2);
  }
  return launch_status();
}

int kv_write(const uint16_t* k, const uint16_t* v, uint8_t* k_cache, uint8_t* v_cache,
             const int64_t* slot_mapping, int32_t num_tokens, int32_t heads, int32_t head_dim,
             int32_t block_size, int64_t num_blocks, float k_scale, float v_scale,
             int64_t key_stride, int64_t value_stride, int64_t cache_stride,
             hipStream_t stream, float* amax2) {
  const int64_t e = int64_t(heads) * head_dim;
  const int64_t nslots = num_blocks * block_size;
  // reciprocals on the host: IEEE binary32 division, RN(1/scale)
  const float k_inv = 1.0f / k_scale, v_inv = 1.0f / v_scale;
  const bool wide = e % 16 == 0 && e <= 512 && 64 % (2 * (e / 16)) == 0 &&
                    key_stride % 8 == 0 && value_stride % 8 == 0 && cache_stride % 16 == 0 &&
                    aligned(k, 16) && aligned(v, 16) && aligned(k_cache, 16) &&
                    aligned(v_cache, 16);
  if (wide) {
    const int lpt = int(e / 16);
    const int lpt_log2 = __builtin_ctz(unsigned(lpt));
    const int64_t per_block = int64_t(kWideBlock / 64) * (64 / (2 * lpt));
    const int64_t blocks = clamp_grid((int64_t(num_tokens) + per_block - 1) / per_block);
    if (amax2)
      launch(kv_write_wide_kernel<true>, dim3(unsigned(blocks)), dim3(kWideBlock), 0, stream,
             k, v, k_cache, v_cache, slot_mapping, int64_t(num_tokens), lpt_log2, key_stride,
             value_stride, cache_stride, block_size, nslots, k_scale, k_inv, v_scale, v_inv,
             amax2);
    else
      launch(kv_write_wide_kernel<false>, dim3(unsigned(blocks)), dim3(kWideBlock), 0, stream,
             k, v, k_cache, v_cache, slot_mapping, int64_t(num_tokens), lpt_log2, key_stride,
             value_stride, cache_stride, block_size, nslots, k_scale, k_inv, v_scale, v_inv,
             amax2);
    return launch_status();
  }
  if (amax2) {  // other geometries: the absmax pass, then the write
    const int rc = kv_amax_rows(k, v, num_tokens, e, key_stride, value_stride, amax2, stream);
    if (rc != FP8Q_OK) return rc;
  }
  const bool vec = e % 8 == 0 && key_stride % 8 == 0 && value_stride % 8 == 0 &&
                   cache_stride % 8 == 0 && aligned(k, 16) && aligned(v, 16) &&
                   aligned(k_cache, 8) && aligned(v_cache, 8);
  const int64_t rows_per_block = vec ? kRowsPerBlock * kTokPerWave : kRowsPerBlock;
  const int64_t blocks = clamp_grid((int64_t(num_tokens) + rows_per_block - 1) / rows_per_block);
  if (vec)
    launch(kv_write_vec_kernel, dim3(unsigned(blocks)), dim3(64, kRowsPerBlock), 0,
                       stream, reinterpret_cast<const uint4*>(k),
                       reinterpret_cast<const uint4*>(v), reinterpret_cast<uint2*>(k_cache),
                       reinterpret_cast<uint2*>(v_cache), slot_mapping, int64_t(num_tokens),
                       int(e / 8), key_stride / 8, value_stride / 8, cache_stride / 8,
                       block_size, nslots, k_scale, k_inv, v_scale, v_inv);
  else
    launch(kv_write_scalar_kernel, dim3(unsigned(blocks)), dim3(64, kRowsPerBlock),
                       0, stream, k, v, k_cache, v_cache, slot_mapping, int64_t(num_tokens),
                       int(e), key_stride, value_stride, cache_stride, block_size, nslots,
                       k_scale, k_inv, v_scale, v_inv);
  return launch_status();
}

int kv_last_writer_slots(const int64_t* slots, int64_t* out, int32_t n, hipStream_t stream) {
  if (n <= 0) return FP8Q_OK;
  if (n > 65535 * 64) return FP8Q_EINVAL;
  if (hipMemcpyAsync(out, slots, size_t(n) * sizeof(int64_t), hipMemcpyDeviceToDevice,
                     stream) != hipSuccess)
    return FP8Q_EHIP;
  const unsigned tiles = unsigned((n + 63) / 64);
  launch(kv_mark_superseded_kernel, dim3(tiles, tiles), dim3(64), 0, stream, slots, out, n);
  return launch_status();
}

static int kv_read(const uint8_t* k_cache, const uint8_t* v_cache, const int64_t* slot_mapping,
            int32_t num_tokens, int32_t heads, int32_t head_dim, int32_t block_size,
            int64_t num_blocks, float k_scale, float v_scale, uint16_t* k_out,
            uint16_t* v_out, int64_t out_key_stride, int64_t out_value_stride,
            int64_t cache_stride, hipStream_t stream) {
  const int64_t e = int64_t(heads) * head_dim;
  const int64_t nslots = num_blocks * block_size;
  const bool vec = e % 8 == 0 && out_key_stride % 8 == 0 && out_value_stride % 8 == 0 &&
                   cache_stride % 8 == 0 && aligned(k_cache, 8) && aligned(v_cache, 8) &&
                   aligned(k_out, 16) && aligned(v_out, 16) && e / 8 <= 0x7FFFFFFF;
  if (vec) {
    const int64_t items = int64_t(num_tokens) * (e / 8);
    const int64_t per_block = int64_t(kReadBlock) * kReadUnroll;
    const int64_t blocks = clamp_grid((items + per_block - 1) / per_block);
    // 32-bit indices when no item index the loop forms (< 2 * items + per_block) and no
    // slot can wrap
    const uint32_t ipt = uint32_t(e / 8);
    const bool pow2 = (ipt & (ipt - 1)) == 0;
    const uint32_t ipt_log2 = uint32_t(__builtin_ctz(ipt));
    if (items < (int64_t(1) << 31) - per_block && nslots <= 0x7FFFFFFF) {
      auto kern = pow2 ? kv_read_vec_kernel<uint32_t, true> : kv_read_vec_kernel<uint32_t, false>;
      launch(kern, dim3(unsigned(blocks)), dim3(kReadBlock), 0, stream, k_cache, v_cache,
             slot_mapping, uint32_t(items), ipt, ipt_log2, cache_stride, uint32_t(block_size),
             nslots, k_scale, v_scale, k_out, v_out, out_key_stride, out_value_stride);
    } else {
      auto kern = pow2 ? kv_read_vec_kernel<uint64_t, true> : kv_read_vec_kernel<uint64_t, false>;
      launch(kern, dim3(unsigned(blocks)), dim3(kReadBlock), 0, stream, k_cache, v_cache,
             slot_mapping, uint64_t(items), ipt, ipt_log2, cache_stride, uint32_t(block_size),
             nslots, k_scale, v_scale, k_out, v_out, out_key_stride, out_value_stride);
    }
    return launch_status();
  }
  if (e > 0x7FFFFFFF) return FP8Q_EINVAL;
  const int64_t blocks =
      clamp_grid((int64_t(num_tokens) + kRowsPerBlock - 1) / kRowsPerBlock);
  launch(kv_read_scalar_kernel, dim3(unsigned(blocks)), dim3(64, kRowsPerBlock), 0, stream,
         k_cache, v_cache, slot_mapping, int64_t(num_tokens), int(e), cache_stride,
         block_size, nslots, k_scale, v_scale, k_out, v_out, out_key_stride,
         out_value_stride);
  return launch_status();
}

}  // namespace fp8q

using namespace fp8q;

extern "C" int fp8_kv_write(const uint16_t* k, const uint16_t* v, uint8_t* k_cache,
                            uint8_t* v_cache, const int64_t* slot_mapping, int32_t num_tokens,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int64_t num_blocks, float k_scale, float v_scale,
                            int32_t key_stride, int32_t value_stride, int64_t cache_stride,
                            hipStream_t stream) {
  const int rc = kv_write_check(num_tokens, num_kv_heads, head_dim, block_size, num_blocks,
                                k_scale, v_scale, key_stride, value_stride, cache_stride);
  if (rc != FP8Q_OK) return rc;
  if (num_tokens == 0) return FP8Q_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping) return FP8Q_ENULL;
  if (!aligned(slot_mapping, 8)) return FP8Q_EALIGN;
  return kv_write(k, v, k_cache, v_cache, slot_mapping, num_tokens, num_kv_heads, head_dim,
                  block_size, num_blocks, k_scale, v_scale, key_stride, value_stride,
                  cache_stride, stream);
}

extern "C" int fp8_kv_write_amax(const uint16_t* k, const uint16_t* v, uint8_t* k_cache,
                                 uint8_t* v_cache, const int64_t* slot_mapping,
                                 int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int64_t num_blocks, float k_scale,
                                 float v_scale, int32_t key_stride, int32_t value_stride,
                                 int64_t cache_stride, float* amax2, hipStream_t stream) {
  const int rc = kv_write_check(num_tokens, num_kv_heads, head_dim, block_size, num_blocks,
                                k_scale, v_scale, key_stride, value_stride, cache_stride);
  if (rc != FP8Q_OK) return rc;
  if (num_tokens == 0) return FP8Q_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping || !amax2) return FP8Q_ENULL;
  if (!aligned(slot_mapping, 8) || !aligned(amax2, 4)) return FP8Q_EALIGN;
  return kv_write(k, v, k_cache, v_cache, slot_mapping, num_tokens, num_kv_heads, head_dim,
                  block_size, num_blocks, k_scale, v_scale, key_stride, value_stride,
                  cache_stride, stream, amax2);
}

extern "C" int fp8_kv_amax(const uint16_t* k, const uint16_t* v, int64_t n_elems,
                           float* amax2, hipStream_t stream) {
  if (n_elems < 0) return FP8Q_EINVAL;
  if (n_elems == 0) return FP8Q_OK;
  if (!k || !v || !amax2) return FP8Q_ENULL;
  if (!aligned(amax2, 4)) return FP8Q_EALIGN;
  return kv_amax_rows(k, v, 1, n_elems, n_elems, n_elems, amax2, stream);
}

extern "C" int fp8_kv_read(const uint8_t* k_cache, const uint8_t* v_cache,
                           const int64_t* slot_mapping, int32_t num_tokens,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int64_t num_blocks, float k_scale, float v_scale, uint16_t* k_out,
                           uint16_t* v_out, int32_t out_key_stride, int32_t out_value_stride,
                           int64_t cache_stride, hipStream_t stream) {
  const int rc = kv_write_check(num_tokens, num_kv_heads, head_dim, block_size, num_blocks,
                                k_scale, v_scale, out_key_stride, out_value_stride,
                                cache_stride);
  if (rc != FP8Q_OK) return rc;
  if (num_tokens == 0) return FP8Q_OK;
  if (!k_cache || !v_cache || !slot_mapping || !k_out || !v_out) return FP8Q_ENULL;
  if (!aligned(slot_mapping, 8) || !aligned(k_out, 2) || !aligned(v_out, 2))
    return FP8Q_EALIGN;
  return kv_read(k_cache, v_cache, slot_mapping, num_tokens, num_kv_heads, head_dim,
                 block_size, num_blocks, k_scale, v_scale, k_out, v_out, out_key_stride,
                 out_value_stride, cache_stride, stream);
}
