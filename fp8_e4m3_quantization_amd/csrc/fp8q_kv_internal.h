// fp8q_kv_internal.h -- KV helpers shared by the C-ABI entry points and the calibrator.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fp8q.h"

namespace fp8q {

// Argument checks of fp8_kv_write that need no pointer (CPU-testable; nothing enqueued).
inline int kv_write_check(int32_t num_tokens, int32_t heads, int32_t head_dim,
                          int32_t block_size, int64_t num_blocks, float k_scale,
                          float v_scale, int64_t key_stride, int64_t value_stride,
                          int64_t cache_stride) {
  if (num_tokens < 0 || heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return FP8Q_EINVAL;
  const int64_t e = int64_t(heads) * head_dim;
  if (key_stride < e || value_stride < e) return FP8Q_EINVAL;
  if (cache_stride < int64_t(block_size) * e) return FP8Q_EINVAL;
  if (num_blocks > (int64_t(1) << 62) / cache_stride) return FP8Q_EINVAL;
  // scales in [2^-64, 2^64] keep every step of the reciprocal-based exact division in
  // the normal binary32 range (NaN fails both comparisons)
  if (!(k_scale >= 0x1p-64f && k_scale <= 0x1p64f) ||
      !(v_scale >= 0x1p-64f && v_scale <= 0x1p64f))
    return FP8Q_EINVAL;
  return FP8Q_OK;
}

int kv_write(const uint16_t* k, const uint16_t* v, uint8_t* k_cache, uint8_t* v_cache,
             const int64_t* slot_mapping, int32_t num_tokens, int32_t heads, int32_t head_dim,
             int32_t block_size, int64_t num_blocks, float k_scale, float v_scale,
             int64_t key_stride, int64_t value_stride, int64_t cache_stride,
             hipStream_t stream, float* amax2 = nullptr);

// out = slots with -1 in place of every token that a later token of the list overwrites
// (the same slot); the survivors are distinct, so one kv_write of the whole list leaves the
// pools exactly as writing the list's tokens one after another would.
int kv_last_writer_slots(const int64_t* slots, int64_t* out, int32_t n, hipStream_t stream);

// A calibration batch staged in one pass: rows copied packed to dk / dv, slots to dslots,
// the rows' |K| / |V| maxima folded into amax2 (one kernel for 16-byte aligned geometries,
// else the absmax pass and copies).
int kv_stage(const uint16_t* k, const uint16_t* v, const int64_t* slots, int64_t rows,
             int64_t e, int64_t key_stride, int64_t value_stride, uint16_t* dk, uint16_t* dv,
             int64_t* dslots, float* amax2, hipStream_t stream);

int kv_amax_rows(const uint16_t* k, const uint16_t* v, int64_t rows, int64_t row_elems,
                 int64_t key_stride, int64_t value_stride, float* amax2, hipStream_t stream);

}  // namespace fp8q
