// fp8q_calib.hip -- online per-tensor FP8 KV scale calibration for one attention layer
// (host object behind the C ABI; its device work goes through a table of callbacks, by
// default the library's own HIP kernels and copies).
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
// Both pages hand the calibrator a GPU backend object; here that is fp8q_kv_calib_ops, so
// the bookkeeping below never touches device memory and runs unchanged against a table
// backed by host memory.
//
// Differences from the pages: the pages synchronize the stream on every observe inside
// the window to read the batch's absmax back, and stage with separate copies.  Here the
// running maximum is max-accumulated on the device across the whole window and read once,
// at the freeze;
// max is order-free, so the frozen scales are bit-identical.  The pages replay one write
// per staged batch, in order; the HIP table's replay is one write of all staged tokens
// after dropping every token a later staged token overwrites (last writer wins either
// way, so the pool bytes are the same).  The staging is one stream-ordered allocation,
// released in stream order, so the freeze blocks only for the 8-byte read; an in-window
// observe is one kernel (the batch's absmax and its staging copy in one pass).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

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
constexpr float kAmaxFloor = 1e-10f;

// Scales the write accepts (the range of its exact reciprocal division).
bool scale_in_range(float s) { return s >= 0x1p-64f && s <= 0x1p64f; }

// ------------------------------------------------------------------ HIP callbacks
struct HipCtx {
  int device = -1;
};

// 64 bytes of page-locked host memory for the freezes' reads, shared by every calibrator of
// the process (allocated at the first freeze, kept until the process ends; reads take turns).
std::mutex g_pinned_mu;
void* g_pinned = nullptr;

// Clears `n` bytes with a kernel rather than a memset node, so that the calibrator's device
// work holds no memset if a caller ever captures it.
__global__ __launch_bounds__(64) void zero_bytes_kernel(uint8_t* p, uint64_t n) {
  for (uint64_t i = threadIdx.x; i < n; i += 64) p[i] = 0;
}

int hip_device(void* ctx, int32_t* dev) {
  int d = 0;
  if (hipGetDevice(&d) != hipSuccess) return FP8Q_EHIP;
  static_cast<HipCtx*>(ctx)->device = d;
  *dev = d;
  return FP8Q_OK;
}

int hip_alloc(void*, uint64_t bytes, void** out, hipStream_t stream) {
  *out = nullptr;
  if (hipMallocAsync(out, size_t(bytes), stream) != hipSuccess) {
    *out = nullptr;
    return FP8Q_EHIP;
  }
  return FP8Q_OK;
}

int hip_release(void* ctx, void* p, hipStream_t stream, int32_t at_destroy) {
  if (!p) return FP8Q_OK;
  if (!at_destroy) return hipFreeAsync(p, stream) == hipSuccess ? FP8Q_OK : FP8Q_EHIP;
  // destroy: no stream to order against, so wait for the owning device to go idle first
  const int dev = static_cast<HipCtx*>(ctx)->device;
  int prev = 0;
  const bool have_prev = hipGetDevice(&prev) == hipSuccess;
  if (dev >= 0) (void)hipSetDevice(dev);
  int rc = FP8Q_OK;
  if (hipDeviceSynchronize() != hipSuccess || hipFreeAsync(p, nullptr) != hipSuccess ||
      hipStreamSynchronize(nullptr) != hipSuccess)
    rc = FP8Q_EHIP;
  if (have_prev) (void)hipSetDevice(prev);
  return rc;
}

int hip_zero(void*, void* p, uint64_t bytes, hipStream_t stream) {
  if (bytes == 0) return FP8Q_OK;
  fp8q::launch(zero_bytes_kernel, dim3(1), dim3(64), 0, stream, static_cast<uint8_t*>(p),
               bytes);
  return fp8q::launch_status();
}

int hip_amax_rows(void*, const uint16_t* k, const uint16_t* v, int64_t rows, int64_t elems,
                  int64_t ks, int64_t vs, float* amax2, hipStream_t stream) {
  return fp8q::kv_amax_rows(k, v, rows, elems, ks, vs, amax2, stream);
}

// staging.rs page, copy_rows: one linear copy when the source rows are packed, else a 2-D
// copy of `rows` rows of row_bytes from a pitch of src_pitch bytes.
int hip_copy2d(void*, void* dst, const void* src, int64_t src_pitch, int64_t row_bytes,
               int64_t rows, hipStream_t stream) {
  hipError_t e;
  if (src_pitch == row_bytes)
    e = hipMemcpyAsync(dst, src, size_t(row_bytes) * size_t(rows), hipMemcpyDeviceToDevice,
                       stream);
  else
    e = hipMemcpy2DAsync(dst, size_t(row_bytes), src, size_t(src_pitch), size_t(row_bytes),
                         size_t(rows), hipMemcpyDeviceToDevice, stream);
  return e == hipSuccess ? FP8Q_OK : FP8Q_EHIP;
}

int hip_stage(void*, const uint16_t* k, const uint16_t* v, const int64_t* slots, int64_t rows,
              int64_t elems, int64_t ks, int64_t vs, uint16_t* dk, uint16_t* dv, int64_t* dslots,
              float* amax2, hipStream_t stream) {
  return fp8q::kv_stage(k, v, slots, rows, elems, ks, vs, dk, dv, dslots, amax2, stream);
}

// The one blocking read: into page-locked memory (a direct copy, where pageable memory is
// staged through the runtime's own buffer), then to the caller's memory.
int hip_read(void*, void* host_dst, const void* src, uint64_t bytes, hipStream_t stream) {
  std::lock_guard<std::mutex> lock(g_pinned_mu);
  if (bytes <= 64 && !g_pinned && hipHostMalloc(&g_pinned, 64, hipHostMallocDefault) != hipSuccess)
    g_pinned = nullptr;
  void* dst = (bytes <= 64 && g_pinned) ? g_pinned : host_dst;
  if (hipMemcpyAsync(dst, src, size_t(bytes), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return FP8Q_EHIP;
  if (dst != host_dst) memcpy(host_dst, dst, size_t(bytes));
  return FP8Q_OK;
}

// One write of every staged token, in place of one write per staged batch in order:
// tokens that a later staged token overwrites are dropped first, so every slot gets the
// bytes of its last staged writer -- what the ordered replay leaves.  Staged rows are
// packed: one row of `elems` per token, whatever the live strides.
int hip_replay(void*, const uint16_t* k, const uint16_t* v, const int64_t* slots,
               int64_t* scratch_slots, int32_t n, int32_t elems, const fp8q_kv_target* t,
               float k_scale, float v_scale, hipStream_t stream) {
  int rc = fp8q::kv_last_writer_slots(slots, scratch_slots, n, stream);
  if (rc != FP8Q_OK) return rc;
  return fp8q::kv_write(k, v, t->k_pool, t->v_pool, scratch_slots, n, 1, elems,
                        t->block_size, t->num_blocks, k_scale, v_scale, elems, elems,
                        t->cache_stride, stream);
}

}  // namespace

struct fp8q_kv_calib {
  std::mutex mu;
  fp8q_kv_calib_ops ops = {};
  HipCtx hip;  // the HIP table's context (unused with a caller's table)
  int32_t window = 0, requested = 0;
  float headroom = 1.0f, provisional = 2.0f;
  int64_t tokens_seen = 0, unstaged = 0, replayed = 0;
  int32_t staged_batches = 0;  // batches staged over the window (kept after the freeze)
  bool frozen = false;
  float k_scale = 2.0f, v_scale = 2.0f;
  float k_amax = 0.0f, v_amax = 0.0f;
  int32_t device = -1;
  float* d_amax = nullptr;  // device float[2]: running max |K|, |V| over the window
  // staging: packed bf16 rows and int64 slots of every staged batch, in order, carved from
  // one allocation (base)
  void* base = nullptr;
  uint16_t* sk = nullptr;
  uint16_t* sv = nullptr;
  int64_t* sslots = nullptr;
  int64_t* rslots = nullptr;  // replay scratch: int64 [capacity]
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

// Releases the staging (staging.rs page, KvStaging::release; idempotent).
int release_staging(fp8q_kv_calib* c, hipStream_t stream, int32_t at_destroy) {
  const int rc = c->base ? c->ops.release(c->ops.ctx, c->base, stream, at_destroy) : FP8Q_OK;
  c->base = nullptr;
  c->sk = c->sv = nullptr;
  c->sslots = c->rslots = nullptr;
  c->capacity = c->elems = c->used = 0;
  c->batches.clear();
  return rc;
}

// Byte offsets of the four staging regions for `rows` tokens of `e` elements, each 256-byte
// aligned: K rows, V rows, slots, replay scratch; [4] is the total.
void staging_layout(uint64_t rows, uint64_t e, uint64_t off[5]) {
  const auto up = [](uint64_t b) { return (b + 255) & ~uint64_t(255); };
  off[0] = 0;
  off[1] = off[0] + up(rows * e * 2);
  off[2] = off[1] + up(rows * e * 2);
  off[3] = off[2] + up(rows * 8);
  off[4] = off[3] + up(rows * 8);
}

float freeze_scale(float amax, float headroom) {
  const float a = amax > kAmaxFloor ? amax : kAmaxFloor;
  return (a * headroom) / 448.0f;
}

int create(int32_t window_tokens, float headroom, float provisional_scale,
           const fp8q_kv_calib_ops* ops, fp8q_kv_calib** out) {
  if (!out) return FP8Q_ENULL;
  *out = nullptr;
  if (window_tokens <= 0 || !isfinite(headroom) || headroom > 0x1p64f ||
      !scale_in_range(provisional_scale))
    return FP8Q_EINVAL;
  if (ops && (!ops->device || !ops->alloc || !ops->release || !ops->zero || !ops->amax_rows ||
              !ops->copy2d || !ops->read || !ops->replay))
    return FP8Q_ENULL;
  fp8q_kv_calib* c = new (std::nothrow) fp8q_kv_calib();
  if (!c) return FP8Q_EHIP;
  if (ops) {
    c->ops = *ops;
  } else {
    c->ops = fp8q_kv_calib_ops{&c->hip,       hip_device, hip_alloc, hip_release,
                               hip_zero,       hip_amax_rows, hip_copy2d, hip_read,
                               hip_replay,     hip_stage};
  }
  c->requested = window_tokens;
  c->window = window_tokens < kMaxStagedTokens ? window_tokens : kMaxStagedTokens;
  c->headroom = headroom >= 1.0f ? headroom : 1.0f;
  c->provisional = provisional_scale;
  c->k_scale = c->v_scale = provisional_scale;
  *out = c;
  return FP8Q_OK;
}

}  // namespace

extern "C" int fp8q_kv_calib_create(int32_t window_tokens, float headroom,
                                    float provisional_scale, fp8q_kv_calib** out) {
  return create(window_tokens, headroom, provisional_scale, nullptr, out);
}

extern "C" int fp8q_kv_calib_create_with_ops(int32_t window_tokens, float headroom,
                                             float provisional_scale,
                                             const fp8q_kv_calib_ops* ops,
                                             fp8q_kv_calib** out) {
  if (!ops) return FP8Q_ENULL;
  return create(window_tokens, headroom, provisional_scale, ops, out);
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
  int rc = fp8q::kv_write_check(num_tokens, num_kv_heads, head_dim, t->block_size,
                                t->num_blocks, c->provisional, c->provisional, t->key_stride,
                                t->value_stride, t->cache_stride);
  if (rc != FP8Q_OK) return rc;
  if (num_tokens == 0) return FP8Q_OK;
  if (!k || !v || !t->k_pool || !t->v_pool || !t->slot_mapping) return FP8Q_ENULL;
  const int64_t n = num_tokens, e = int64_t(num_kv_heads) * head_dim;
  const fp8q_kv_calib_ops& ops = c->ops;

  std::lock_guard<std::mutex> lock(c->mu);
  if (c->frozen) return FP8Q_OK;
  int32_t dev = 0;
  rc = ops.device(ops.ctx, &dev);
  if (rc != FP8Q_OK) return rc;
  if (!c->d_amax) {
    void* p = nullptr;
    rc = ops.alloc(ops.ctx, 2 * sizeof(float), &p, stream);
    if (rc != FP8Q_OK) return rc;
    rc = ops.zero(ops.ctx, p, 2 * sizeof(float), stream);
    if (rc != FP8Q_OK) {
      (void)ops.release(ops.ctx, p, stream, 0);
      return rc;
    }
    c->d_amax = static_cast<float*>(p);
    c->device = dev;
  } else if (dev != c->device) {
    return FP8Q_ESTATE;
  }

  const int step = decide_locked(c, n, e);
  // allocate before touching any state, so a failure leaves the calibrator unchanged
  if (step == FP8Q_CALIB_STAGE && c->capacity == 0) {
    uint64_t off[5];
    staging_layout(uint64_t(c->window), uint64_t(e), off);
    void* p = nullptr;
    rc = ops.alloc(ops.ctx, off[4], &p, stream);
    if (rc != FP8Q_OK) return rc;
    uint8_t* b = static_cast<uint8_t*>(p);
    c->base = p;
    c->sk = reinterpret_cast<uint16_t*>(b + off[0]);
    c->sv = reinterpret_cast<uint16_t*>(b + off[1]);
    c->sslots = reinterpret_cast<int64_t*>(b + off[2]);
    c->rslots = reinterpret_cast<int64_t*>(b + off[3]);
    c->capacity = c->window;
    c->elems = e;
  }

  if (step == FP8Q_CALIB_STAGE) {
    uint16_t* dk = c->sk + c->used * c->elems;
    uint16_t* dv = c->sv + c->used * c->elems;
    if (ops.stage) {
      rc = ops.stage(ops.ctx, k, v, t->slot_mapping, n, e, t->key_stride, t->value_stride, dk,
                     dv, c->sslots + c->used, c->d_amax, stream);
    } else {
      rc = ops.amax_rows(ops.ctx, k, v, n, e, t->key_stride, t->value_stride, c->d_amax,
                         stream);
      if (rc == FP8Q_OK)
        rc = ops.copy2d(ops.ctx, dk, k, int64_t(t->key_stride) * 2, e * 2, n, stream);
      if (rc == FP8Q_OK)
        rc = ops.copy2d(ops.ctx, dv, v, int64_t(t->value_stride) * 2, e * 2, n, stream);
      if (rc == FP8Q_OK)
        rc = ops.copy2d(ops.ctx, c->sslots + c->used, t->slot_mapping, n * 8, n * 8, 1, stream);
    }
    if (rc != FP8Q_OK) return rc;
    c->tokens_seen += n;
    c->batches.emplace_back(c->used, int32_t(n));
    c->staged_batches += 1;
    c->used += n;
    return FP8Q_OK;
  }

  rc = ops.amax_rows(ops.ctx, k, v, n, e, t->key_stride, t->value_stride, c->d_amax, stream);
  if (rc != FP8Q_OK) return rc;
  if (step == FP8Q_CALIB_DECLINE) {
    c->tokens_seen += n;
    c->unstaged += n;
    return FP8Q_OK;
  }

  // FREEZE: read the window's running maxima once, then rewrite the staged batches.
  float host_amax[2] = {0.0f, 0.0f};
  rc = ops.read(ops.ctx, host_amax, c->d_amax, sizeof(host_amax), stream);
  if (rc != FP8Q_OK) return rc;
  const float ks = freeze_scale(host_amax[0], c->headroom);
  const float vs = freeze_scale(host_amax[1], c->headroom);
  if (!scale_in_range(ks) || !scale_in_range(vs)) return FP8Q_EINVAL;
  if (c->used > 0) {
    rc = ops.replay(ops.ctx, c->sk, c->sv, c->sslots, c->rslots, int32_t(c->used),
                    int32_t(c->elems), t, ks, vs, stream);
    if (rc != FP8Q_OK) return rc;
  }
  c->k_amax = host_amax[0];
  c->v_amax = host_amax[1];
  c->k_scale = ks;
  c->v_scale = vs;
  c->frozen = true;
  c->tokens_seen += n;
  c->replayed = c->used;
  // stream-ordered: the release happens after the replay, and observe returns without
  // waiting for it
  return release_staging(c, stream, 0);
}

extern "C" int fp8q_kv_calib_scales(const fp8q_kv_calib* c, float* k_scale, float* v_scale) {
  if (!c || !k_scale || !v_scale) return FP8Q_ENULL;
  std::lock_guard<std::mutex> lock(const_cast<fp8q_kv_calib*>(c)->mu);
  *k_scale = c->k_scale;
  *v_scale = c->v_scale;
  return FP8Q_OK;
}

extern "C" int fp8q_kv_calib_state(const fp8q_kv_calib* c, fp8q_kv_calib_info* info) {
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
  info->provisional_scale = c->provisional;
  return FP8Q_OK;
}

extern "C" void fp8q_kv_calib_destroy(fp8q_kv_calib* c) {
  if (!c) return;
  (void)release_staging(c, nullptr, 1);
  if (c->d_amax) (void)c->ops.release(c->ops.ctx, c->d_amax, nullptr, 1);
  delete c;
}
