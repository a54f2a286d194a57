// fp8q_calib.hip -- online per-tensor FP8 KV scale calibration for one attention layer
// (host object behind the C ABI; device work goes through the library's own kernels).
//
// fp8_calibration.rs page: module doc (running max of |K| and |V| over the first window
// tokens; the observe that reaches the window freezes scale = amax * headroom / 448 over
// every observed token, its own batch included; the frozen scale is >= amax / 448),
// PROVISIONAL_SCALE (2.0 for writes inside the window), Fp8KvCalibration::new (headroom
// clamped to >= 1, window clamped to MAX_STAGED_TOKENS, window 1 freezes on the first
// observe), ::observe (stage / freeze + replay / frozen), ::absmax.
// staging.rs page: module doc "The fix, and its tradeoff" (option (c): keep the window's
// bf16 K/V and slot mappings and rewrite them through the same write kernel at the frozen
// scale, in write order, so the last writer of every slot is unchanged; the crossing
// batch is written by the caller afterwards), MAX_STAGED_TOKENS = 4096, KvStaging::stage
// (lazy allocation at window capacity; decline when elements per token change or the
// window would overflow), ::replay_and_release (packed strides), ::release, copy_rows.
//
// Differences from the pages: the pages synchronize the stream on every observe inside
// the window to read the batch's absmax back.  Here the running maximum is
// max-accumulated on the device across the whole window and read once, at the freeze;
// max is order-free, so the frozen scales are bit-identical.  The pages replay one write
// per staged batch, in order; here the replay is one write of all staged tokens after
// dropping every token a later staged token overwrites (last writer wins either way, so
// the pool bytes are the same).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <new>
#include <utility>
#include <vector>

#include "fp8q.h"
#include "fp8q_kv_internal.h"
#include "fp8q_launch.h"

#pragma clang fp contract(off)

namespace {
constexpr int32_t kMaxStagedTokens = 4096;
constexpr float kProvisionalScale = 2.0f;
constexpr float kAmaxFloor = 1e-10f;
}  // namespace

struct fp8q_kv_calib {
  std::mutex mu;
  int32_t window = 0, requested = 0;
  float headroom = 1.0f;
  int64_t tokens_seen = 0, unstaged = 0, replayed = 0;
  int32_t staged_batches = 0;  // batches staged over the window (kept after the freeze)
  bool frozen = false;
  float k_scale = kProvisionalScale, v_scale = kProvisionalScale;
  float k_amax = 0.0f, v_amax = 0.0f;
  int device = -1;
  float* d_amax = nullptr;  // device float[2]: running max |K|, |V| over the window
  // staging: packed bf16 rows and int64 slots of every staged batch, in order
  uint16_t* sk = nullptr;
  uint16_t* sv = nullptr;
  int64_t* sslots = nullptr;
  int64_t* rslots = nullptr;  // replay slots: sslots with overwritten tokens set to -1
  int64_t capacity = 0, elems = 0, used = 0;
  std::vector<std::pair<int64_t, int32_t>> batches;  // (offset tokens, tokens)
};

namespace {

int decide_locked(const fp8q_kv_calib* c, int64_t n, int64_t e) {
  if (c->frozen) return FP8Q_CALIB_FROZEN;
  if (c->tokens_seen + n >= c->window) return FP8Q_CALIB_FREEZE;
  if (c->capacity != 0 && (e != c->elems || c->used + n > c->capacity))
    return FP8Q_CALIB_DECLINE;
  return FP8Q_CALIB_STAGE;
}

void release_staging(fp8q_kv_calib* c) {
  if (c->sk) (void)hipFree(c->sk);
  if (c->sv) (void)hipFree(c->sv);
  if (c->sslots) (void)hipFree(c->sslots);
  if (c->rslots) (void)hipFree(c->rslots);
  c->sk = c->sv = nullptr;
  c->sslots = c->rslots = nullptr;
  c->capacity = c->elems = c->used = 0;
  c->batches.clear();
}

// Packed copy of `rows` rows of `e` bf16 from a source with `stride` elements per row.
hipError_t copy_rows(uint16_t* dst, const uint16_t* src, int64_t stride, int64_t e,
                     int64_t rows, hipStream_t s) {
  const size_t row = size_t(e) * 2;
  if (stride == e) return hipMemcpyAsync(dst, src, row * size_t(rows), hipMemcpyDeviceToDevice, s);
  return hipMemcpy2DAsync(dst, row, src, size_t(stride) * 2, row, size_t(rows),
                          hipMemcpyDeviceToDevice, s);
}

float freeze_scale(float amax, float headroom) {
  const float a = amax > kAmaxFloor ? amax : kAmaxFloor;
  return (a * headroom) / 448.0f;
}

}  // namespace

extern "C" int fp8q_kv_calib_create(int32_t window_tokens, float headroom,
                                    fp8q_kv_calib** out) {
  if (!out) return FP8Q_ENULL;
  *out = nullptr;
  if (window_tokens <= 0 || !isfinite(headroom)) return FP8Q_EINVAL;
  fp8q_kv_calib* c = new (std::nothrow) fp8q_kv_calib();
  if (!c) return FP8Q_EHIP;
  c->requested = window_tokens;
  c->window = window_tokens < kMaxStagedTokens ? window_tokens : kMaxStagedTokens;
  c->headroom = headroom >= 1.0f ? headroom : 1.0f;
  *out = c;
  return FP8Q_OK;
}

extern "C" int fp8q_kv_calib_decide(const fp8q_kv_calib* c, int32_t num_tokens,
                                    int32_t elems_per_token) {
  if (!c) return FP8Q_ENULL;
  if (num_tokens < 0 || elems_per_token <= 0) return FP8Q_EINVAL;
  std::lock_guard<std::mutex> lock(const_cast<fp8q_kv_calib*>(c)->mu);
  return decide_locked(c, num_tokens, elems_per_token);
}

extern "C" int fp8q_kv_calib_observe(fp8q_kv_calib* c, const uint16_t* k, const uint16_t* v,
                                     int32_t num_tokens, int32_t num_kv_heads,
                                     int32_t head_dim, const fp8q_kv_target* t,
                                     hipStream_t stream) {
  if (!c || !t) return FP8Q_ENULL;
  const int rc = fp8q::kv_write_check(num_tokens, num_kv_heads, head_dim, t->block_size,
                                      t->num_blocks, kProvisionalScale, kProvisionalScale,
                                      t->key_stride, t->value_stride, t->cache_stride);
  if (rc != FP8Q_OK) return rc;
  if (num_tokens == 0) return FP8Q_OK;
  if (!k || !v || !t->k_pool || !t->v_pool || !t->slot_mapping) return FP8Q_ENULL;
  const int64_t n = num_tokens, e = int64_t(num_kv_heads) * head_dim;

  std::lock_guard<std::mutex> lock(c->mu);
  if (c->frozen) return FP8Q_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FP8Q_EHIP;
  if (!c->d_amax) {
    if (hipMalloc(&c->d_amax, 2 * sizeof(float)) != hipSuccess) {
      c->d_amax = nullptr;
      return FP8Q_EHIP;
    }
    c->device = dev;
    if (hipMemsetAsync(c->d_amax, 0, 2 * sizeof(float), stream) != hipSuccess)
      return FP8Q_EHIP;
  } else if (dev != c->device) {
    return FP8Q_ESTATE;
  }

  const int step = decide_locked(c, n, e);
  // allocate before touching any state, so a failure leaves the calibrator unchanged
  if (step == FP8Q_CALIB_STAGE && c->capacity == 0) {
    const size_t rows = size_t(c->window);
    if (hipMalloc(&c->sk, rows * size_t(e) * 2) != hipSuccess ||
        hipMalloc(&c->sv, rows * size_t(e) * 2) != hipSuccess ||
        hipMalloc(&c->sslots, rows * sizeof(int64_t)) != hipSuccess ||
        hipMalloc(&c->rslots, rows * sizeof(int64_t)) != hipSuccess) {
      release_staging(c);
      return FP8Q_EHIP;
    }
    c->capacity = c->window;
    c->elems = e;
  }

  int st = fp8q::kv_amax_rows(k, v, n, e, t->key_stride, t->value_stride, c->d_amax, stream);
  if (st != FP8Q_OK) return st;
  c->tokens_seen += n;

  if (step == FP8Q_CALIB_STAGE) {
    uint16_t* dk = c->sk + c->used * c->elems;
    uint16_t* dv = c->sv + c->used * c->elems;
    if (copy_rows(dk, k, t->key_stride, e, n, stream) != hipSuccess ||
        copy_rows(dv, v, t->value_stride, e, n, stream) != hipSuccess ||
        hipMemcpyAsync(c->sslots + c->used, t->slot_mapping, size_t(n) * sizeof(int64_t),
                       hipMemcpyDeviceToDevice, stream) != hipSuccess)
      return FP8Q_EHIP;
    c->batches.emplace_back(c->used, int32_t(n));
    c->staged_batches += 1;
    c->used += n;
    return FP8Q_OK;
  }
  if (step == FP8Q_CALIB_DECLINE) {
    c->unstaged += n;
    return FP8Q_OK;
  }

  // FREEZE: read the window's running maxima once, then rewrite the staged batches.
  float host_amax[2] = {0.0f, 0.0f};
  if (hipMemcpyAsync(host_amax, c->d_amax, sizeof(host_amax), hipMemcpyDeviceToHost,
                     stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return FP8Q_EHIP;
  c->k_amax = host_amax[0];
  c->v_amax = host_amax[1];
  c->k_scale = freeze_scale(c->k_amax, c->headroom);
  c->v_scale = freeze_scale(c->v_amax, c->headroom);
  c->frozen = true;
  if (c->used > 0) {
    // One write of every staged token, in place of one write per staged batch in order:
    // tokens that a later staged token overwrites are dropped first, so every slot gets
    // the bytes of its last staged writer -- what the ordered replay leaves.  Staged rows
    // are packed: one row of `elems` per token, whatever the live strides.
    st = fp8q::kv_last_writer_slots(c->sslots, c->rslots, int32_t(c->used), stream);
    if (st != FP8Q_OK) return st;
    st = fp8q::kv_write(c->sk, c->sv, t->k_pool, t->v_pool, c->rslots, int32_t(c->used), 1,
                        int32_t(c->elems), t->block_size, t->num_blocks, c->k_scale,
                        c->v_scale, c->elems, c->elems, t->cache_stride, stream);
    if (st != FP8Q_OK) return st;
  }
  c->replayed = c->used;
  if (c->capacity != 0) {
    if (hipStreamSynchronize(stream) != hipSuccess) return FP8Q_EHIP;
    release_staging(c);
  }
  return FP8Q_OK;
}

extern "C" int fp8q_kv_calib_scales(const fp8q_kv_calib* c, float* k_scale, float* v_scale) {
  if (!c || !k_scale || !v_scale) return FP8Q_ENULL;
  std::lock_guard<std::mutex> lock(const_cast<fp8q_kv_calib*>(c)->mu);
  *k_scale = c->k_scale;
  *v_scale = c->v_scale;
  return FP8Q_OK;
}

extern "C" int fp8q_kv_calib_get_info(const fp8q_kv_calib* c, fp8q_kv_calib_info* info) {
  if (!c || !info) return FP8Q_ENULL;
  std::lock_guard<std::mutex> lock(const_cast<fp8q_kv_calib*>(c)->mu);
  info->window_tokens = c->window;
  info->requested_tokens = c->requested;
  info->frozen = c->frozen ? 1 : 0;
  info->staged_batches = c->staged_batches;
  info->tokens_seen = c->tokens_seen;
  info->staged_tokens = c->frozen ? c->replayed : c->used;
  info->unstaged_tokens = c->unstaged;
  info->replayed_tokens = c->replayed;
  info->k_scale = c->k_scale;
  info->v_scale = c->v_scale;
  info->k_amax = c->k_amax;
  info->v_amax = c->v_amax;
  info->headroom = c->headroom;
  info->provisional_scale = kProvisionalScale;
  return FP8Q_OK;
}

extern "C" void fp8q_kv_calib_destroy(fp8q_kv_calib* c) {
  if (!c) return;
  if (c->d_amax || c->sk) {
    int prev = 0;
    const bool have_prev = hipGetDevice(&prev) == hipSuccess;
    if (c->device >= 0) (void)hipSetDevice(c->device);
    release_staging(c);
    if (c->d_amax) (void)hipFree(c->d_amax);
    if (have_prev) (void)hipSetDevice(prev);
  }
  delete c;
}
