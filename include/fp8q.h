/*
 * fp8q.h -- C ABI of libfp8q.so: the FP8 (OCP E4M3) quantize-and-consume path on
 * AMD MI355X (gfx950).
 *
 * Conventions for every call
 *   - Device buffers are plain device pointers owned by the caller; the library never
 *     keeps them past the call (the calibrator keeps only its own staging copies).
 *   - bf16 data is passed as its 16-bit pattern (uint16_t), E4M3 codes as uint8_t, scales
 *     as IEEE binary32.  E4M3 is the OCP "FN" encoding: bias 7, no infinities,
 *     S.1111.111 = NaN, largest finite 448.  Encoding is round-to-nearest-even after one
 *     IEEE binary32 division by the scale, saturating to +-448 (never NaN); the sign is
 *     kept, so a negative value that rounds to zero is 0x80.
 *   - Work is enqueued on `stream` (0 = the null stream) and returns without waiting.
 *     No call allocates or synchronizes, except the calibrator as documented.
 *   - Arguments are validated on the host before anything is enqueued; a bad argument
 *     returns a negative FP8Q_E* code and enqueues nothing.  0 means success.  No C++
 *     exception crosses this boundary.
 *
 * Sources (the pages this path comes from, cited by page title and the item on it):
 *   [actq]    spark_model/layers/ops/fp8_act_quant.rs
 *   [decode]  spark_model/layers/ops/dispatch_proj_decode.rs
 *   [staging] spark_model/layers/fp8_calibration/staging.rs
 *   [calib]   metrale_model_layers/layers/fp8_calibration.rs
 *   [resid]   fp8_residency.rs (weight loader page), fp8_twin_bytes
 */
#ifndef FP8Q_H
#define FP8Q_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ----------------------------------------------------------------- status codes */
#define FP8Q_OK 0
#define FP8Q_EINVAL (-1) /* a size, stride or scale outside the contract */
#define FP8Q_ENULL (-2)  /* a required pointer is NULL */
#define FP8Q_EALIGN (-3) /* a pointer or stride breaks the documented alignment */
#define FP8Q_ELAUNCH (-4) /* the kernel launch was rejected by the HIP runtime */
#define FP8Q_EHIP (-5)   /* another HIP runtime call failed (alloc, copy, sync) */
#define FP8Q_ESTATE (-6) /* calibrator used against its contract (e.g. new device) */

/* Human-readable text for a status code (static storage). */
const char* fp8q_strerror(int status);
/* Library version, major*10000 + minor*100 + patch. */
int fp8q_version(void);
/* Measurement hook: the next kernel this host thread enqueues through the library records
 * `start` as it begins executing and `stop` as it completes (hipExtLaunchKernelGGL), so
 * the events' elapsed time is that kernel's own duration.  Either may be NULL.  Every
 * entry point below enqueues exactly one kernel per call, except calls that enqueue
 * nothing (zero sizes, errors) and the calibrator.  Always returns FP8Q_OK. */
int fp8q_time_next_launch(hipEvent_t start, hipEvent_t stop);

/* Measurement references (not steps of the path): kernels that the path's timings are read
 * against, launched through the same hook.  fp8q_reference_empty enqueues one empty
 * 256-thread block (what a launch costs before any work).  fp8q_reference_stream reads
 * src_bytes (a multiple of 16) from src (non-temporal 16-byte loads) and writes
 * src_bytes / 2 to dst -- the 2:1 read/write mix of the group quantizer and the KV write,
 * with no arithmetic -- over a grid of 4 blocks per CU.  src 16-byte and dst 8-byte aligned device memory.
 * fp8q_reference_lds_stream moves total_bytes from src into LDS the way the prefill GEMM
 * moves its operand tiles (16-byte buffer_load ... lds, 64 KB slices, one 512-thread
 * workgroup per CU, one slice landing while the next is issued, a barrier per slice) and
 * nothing else; slice s reads src bytes [(s * 65536) % span_bytes, + 65536).  span_bytes
 * and total_bytes are multiples of 65536, 65536 <= span_bytes <= 0x7FFF0000; src holds
 * span_bytes of device memory, 16-byte aligned.
 * Errors: FP8Q_EINVAL, FP8Q_ENULL, FP8Q_EALIGN, FP8Q_ELAUNCH. */
int fp8q_reference_empty(hipStream_t stream);
int fp8q_reference_stream(const void* src, void* dst, int64_t src_bytes, hipStream_t stream);
int fp8q_reference_lds_stream(const void* src, int64_t span_bytes, int64_t total_bytes,
                              hipStream_t stream);

/* ------------------------------------------------ per-token 1x128 group quant
 * [actq] module doc: one FP32 scale per 128-wide K-group of one token row;
 * [decode] decode_w8a8_quant_act: the activation is quantized once and shared by every
 * projection that reads it, scales in token-major [m, k/128] order.
 *
 * For every row r < m and group g < k/128:
 *   amax = max_j |x[r, 128g + j]|            (exact)
 *   s    = max(amax, 1e-10f) / 448.0f        (binary32, correctly rounded)
 *   scales[r * (k/128) + g] = s
 *   q[r, 128g + j] = E4M3(x[r, 128g + j] / s)
 *
 *   x       device, bf16 [m, k] row-major, 16-byte aligned
 *   q       device, uint8 [m, k] row-major, 16-byte aligned
 *   scales  device, fp32 [m, k/128] row-major, 4-byte aligned
 *   m       rows, 0 <= m (0 is a no-op); m * k < 2^62
 *   k       columns, k > 0 and k % 128 == 0 (the pages' grid is k/128 groups)
 * Errors: FP8Q_EINVAL (k, m), FP8Q_ENULL, FP8Q_EALIGN, FP8Q_ELAUNCH. */
int fp8_group_quant(const uint16_t* x, uint8_t* q, float* scales, int64_t m, int32_t k,
                    hipStream_t stream);

/* ---------------------------------------------- 128x128 weight block quant
 * [decode] module doc, NUMERICS: E4M3 weights carry one FP32 scale per 128x128 block;
 * [resid] fp8_twin_bytes: the grid has ceil(n/128) * ceil(k/128) fp32 entries.
 * The same formula as fp8_group_quant over each 128x128 block (edge blocks clipped):
 *   ws[nb * ceil(k/128) + kb] = max(amax_block, 1e-10f) / 448.0f
 *   wq[i, j] = E4M3(w[i, j] / ws[i/128, j/128])
 *   w   device, bf16 [n, k] row-major; wq device, uint8 [n, k]; ws device, fp32 grid
 *   n, k > 0.  A preparation utility (weights arrive pre-quantized on the pages).
 * Errors: FP8Q_EINVAL, FP8Q_ENULL, FP8Q_ELAUNCH. */
int fp8_block_quant(const uint16_t* w, uint8_t* wq, float* ws, int32_t n, int32_t k,
                    hipStream_t stream);

/* -------------------------------------------- element-wise binary32 -> E4M3
 * The encoder every kernel above uses, exposed on its own: q[i] = E4M3(x[i]) for finite
 * x, round-to-nearest-even, saturating to +-448 (no scale).
 *   x device fp32 [n], q device uint8 [n], n >= 0.  Errors: FP8Q_EINVAL, FP8Q_ENULL,
 *   FP8Q_ELAUNCH. */
int fp8_e4m3_encode(const float* x, uint8_t* q, int64_t n, hipStream_t stream);

/* ----------------------------------------------- block-scaled W8A8 decode GEMM
 * [decode] decode_w8a8_gemm and module doc NUMERICS: out = act_fp8 @ weight^T with the
 * per-token 1x128 activation scales and the 128x128 weight block scales folded in an
 * FP32 epilogue; DecodeW8a8Plan / decode_w8a8_selected: n % 128 == 0, k % 128 == 0,
 * ldc >= n; DECODE_W8A8_ROWS: the decode band is up to 16 rows; strided_out_extent_elems:
 * a call touches (rows - 1) * ldc + n elements of `out`.
 *
 *   out[r, c] = bf16_rne( sum_g a_scale[r, g] * w_scale[c/128, g]
 *                                * sum_{j<128} dec(a_q[r, 128g+j]) * dec(w_q[c, 128g+j]) )
 * with FP32 products and accumulation.  Only rows 0..m-1 are written: exactly the
 * (m - 1) * ldc + n elements starting at `out`, columns n..ldc-1 of each row untouched.
 *
 *   a_q      device, uint8 [m, k] row-major (E4M3 codes), 16-byte aligned
 *   a_scale  device, fp32 [m, k/128] token-major (fp8_group_quant's own order)
 *   w_q      device, uint8 [n, k] row-major (K contiguous), 16-byte aligned
 *   w_scale  device, fp32 [n/128, k/128]; block (nb, kb) at nb * (k/128) + kb
 *   out      device, bf16 [m, ldc] row-major, 2-byte aligned
 *   1 <= m <= 16; n > 0, n % 128 == 0; k > 0, k % 128 == 0, k <= 131072; ldc >= n.
 * Codes 0x7F/0xFF (NaN) in a_q or w_q propagate NaN into the affected outputs.
 * Errors: FP8Q_EINVAL, FP8Q_ENULL, FP8Q_EALIGN, FP8Q_ELAUNCH. */
int w8a8_block_gemm(const uint8_t* a_q, const float* a_scale, const uint8_t* w_q,
                    const float* w_scale, uint16_t* out, int32_t m, int32_t n, int32_t k,
                    int32_t ldc, hipStream_t stream);

/* ------------------------------------ block-scaled W8A8 decode GEMM, K split
 * [decode] module doc, WHY table: a decode projection is a stream over its weight, and the
 * pages' own library splits K (a split-K pass plus a reduce) when an output alone cannot
 * keep the machine busy.  Computes exactly what w8a8_block_gemm specifies (same operands,
 * layouts, rows written and errors), but when the shape has too few 16-column output
 * strips to give every CU a full share, K is split over `parts` sets of workgroups: each
 * writes its part's FP32 16x16 tile sums to the workspace, and the workgroup that completes
 * a strip adds the parts in a fixed order (p = 0, 1, ...), so the result is deterministic
 * (it may differ from w8a8_block_gemm's in the last bits: another FP32 summation order).
 * Shapes that do not benefit run w8a8_block_gemm's kernel and touch no workspace; K a
 * multiple of 1024 never splits (w8a8_block_gemm's staged form is faster there).
 *
 * w8a8_block_gemm_workspace_size: *bytes = the workspace this shape needs on the current
 *   device (0: no split).  Errors: FP8Q_ENULL, FP8Q_EINVAL (shape as w8a8_block_gemm).
 * w8a8_block_gemm_ws:
 *   workspace        device memory of workspace_bytes >= the size above, 256-byte aligned,
 *                    owned by the caller; its counts (the first ceil(n/16 * 4 / 256) * 256
 *                    bytes) must be zero before the first call that uses it (e.g. zero-filled
 *                    at allocation); every call leaves them zero again, so later calls need
 *                    no clearing.  Calls sharing a workspace must not overlap in time (calls
 *                    on one stream never do).  NULL / 0 is fine when the size is 0.
 * Errors: as w8a8_block_gemm, and FP8Q_ENULL (no workspace where one is needed),
 * FP8Q_EINVAL (workspace_bytes too small), FP8Q_EALIGN (workspace not 256-byte aligned). */
int w8a8_block_gemm_workspace_size(int32_t m, int32_t n, int32_t k, uint64_t* bytes);
int w8a8_block_gemm_ws(const uint8_t* a_q, const float* a_scale, const uint8_t* w_q,
                       const float* w_scale, uint16_t* out, int32_t m, int32_t n, int32_t k,
                       int32_t ldc, void* workspace, uint64_t workspace_bytes,
                       hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, serving
 * loops that forbid allocation): w8a8_block_gemm_ws without the workspace argument.  Same
 * arguments as w8a8_block_gemm and exactly w8a8_block_gemm_ws's result (the same split and
 * summation order), with the split's counts and part tiles in a static device array of
 * 4 KiB + 1 MiB that the library holds on every GPU it runs on until the process ends.
 * Allocates nothing.  The first call on a device looks the array's address up and enqueues
 * a fill that zeroes its counts on `stream`; every call leaves them zero.  All calls on one
 * GPU share the array: calls that overlap in time on one GPU (e.g. on two streams) race;
 * calls on one stream never overlap.  A shape whose split needs more than the array (more
 * than 1024 strips, or strips x parts above 1024) is refused with FP8Q_EINVAL before
 * anything is enqueued; shapes that run unsplit use no scratch.
 * Errors: as w8a8_block_gemm, and FP8Q_EHIP (the array's address could not be looked up). */
int w8a8_block_gemm_noalloc(const uint8_t* a_q, const float* a_scale, const uint8_t* w_q,
                            const float* w_scale, uint16_t* out, int32_t m, int32_t n,
                            int32_t k, int32_t ldc, hipStream_t stream);

/* ------------------------------------------------ W8A8 GEMM at prefill widths
 * [resid] DenseFp8Inputs::w8a8_kernels (the W8A8 prefill arm: per-token group quant, then
 * a block-scaled FP8 GEMM); [actq] module doc (a 4593-token prefill).  The arithmetic and
 * operand layouts are w8a8_block_gemm's; only the row range differs: any m >= 1.  Tiled
 * 256 x 256 (one workgroup per CU) once there are at least half as many such tiles as CUs,
 * else 128 x 128 (two per CU); both tilings give bit-identical results.
 *   out[r, c] = bf16_rne( sum_g a_scale[r, g] * w_scale[c/128, g]
 *                                * sum_{j<128} dec(a_q[r, 128g+j]) * dec(w_q[c, 128g+j]) )
 * FP32 products and accumulation, one scaled FMA per group.  Only rows 0..m-1 are written
 * ((m - 1) * ldc + n elements).
 *   a_q, a_scale, w_q, w_scale, out  as w8a8_block_gemm
 *   m >= 1; n % 128 == 0; k % 128 == 0, 128 * k < 2^31; ldc >= n (16-byte row stores when
 *   ldc % 8 == 0 and out is 16-byte aligned, element stores otherwise).
 * Errors: FP8Q_EINVAL, FP8Q_ENULL, FP8Q_EALIGN, FP8Q_ELAUNCH. */
int w8a8_block_gemm_prefill(const uint8_t* a_q, const float* a_scale, const uint8_t* w_q,
                            const float* w_scale, uint16_t* out, int32_t m, int32_t n,
                            int32_t k, int32_t ldc, hipStream_t stream);

/* ---------------------------------------------- grouped W8A8 decode GEMM
 * [decode] decode_w8a8_quant_act: several projections that read the same activation
 * (attention Q/K/V, a layer's projections) share one quantization; DecodeW8a8Plan::strided:
 * outputs may be written at their own row pitch.  One launch computes, for each
 * projection p < count, exactly what w8a8_block_gemm(a_q, a_scale, projs[p].w_q,
 * projs[p].w_scale, projs[p].out, m, projs[p].n, k, projs[p].ldc) computes (same
 * arithmetic, same bits).  `projs` is host memory read during the call; 1 <= count <= 8;
 * every projection obeys w8a8_block_gemm's rules.  Errors as w8a8_block_gemm. */
typedef struct fp8q_gemm_proj {
  const uint8_t* w_q;    /* device, uint8 [n, k] */
  const float* w_scale;  /* device, fp32 [n/128, k/128] */
  uint16_t* out;         /* device, bf16 [m, ldc] */
  int32_t n;
  int32_t ldc;
} fp8q_gemm_proj;

int w8a8_block_gemm_grouped(const uint8_t* a_q, const float* a_scale,
                            const fp8q_gemm_proj* projs, int32_t count, int32_t m, int32_t k,
                            hipStream_t stream);

/* ------------------------------------- group quant fused into the grouped GEMM
 * [actq] module doc and [decode] decode_w8a8_quant_act + decode_w8a8_gemm, in one launch:
 * the activation is quantized per 1x128 group (exactly fp8_group_quant's arithmetic, so
 * the codes and scales are bit-identical to it) inside the GEMM, each wave quantizing the
 * K-slice it multiplies, then every projection is computed as w8a8_block_gemm_grouped
 * would from those codes (same bits).
 *   a        device, bf16 [m, k] row-major, 16-byte aligned
 *   a_q, a_scale  optional outputs (both NULL or both set): the codes [m, k] and scales
 *            [m, k/128] as fp8_group_quant writes them (16- / 4-byte aligned); required
 *            when k > 8192, where the quantizer and the GEMM run as two launches through
 *            them (FP8Q_ENULL if missing)
 *   projs, count  as w8a8_block_gemm_grouped;  1 <= m <= 16;  k % 128 == 0, k <= 131072
 * Errors: FP8Q_EINVAL, FP8Q_ENULL, FP8Q_EALIGN, FP8Q_ELAUNCH. */
int fp8_quant_w8a8_gemm_grouped(const uint16_t* a, uint8_t* a_q, float* a_scale,
                                const fp8q_gemm_proj* projs, int32_t count, int32_t m,
                                int32_t k, hipStream_t stream);

/* --------------------------------------------- W8A16 decode tier (1..4 rows)
 * [decode] module doc NUMERICS (the W8A16 arithmetic: bf16 activation times E4M3 weight
 * with the same 128x128 FP32 block scales) and DECODE_W8A8_ROWS (up to four rows stay on
 * this tier).  The activation is not quantized:
 *   out[r, c] = bf16_rne( sum_g w_scale[c/128, g] * sum_{j<128} a[r, 128g+j] * dec(w_q[c, 128g+j]) )
 * with exact products and FP32 accumulation (the group's partial, then times its scale).
 * A row's result does not depend on m (the same row gives the same bits at m = 1..4).
 * Only rows 0..m-1 are written ((m - 1) * ldc + n elements).
 *   a        device, bf16 [m, k] row-major, 16-byte aligned
 *   w_q, w_scale, out, n, ldc  as w8a8_block_gemm
 *   1 <= m <= 4; n % 128 == 0; k > 0, k % 128 == 0, k <= 131072; ldc >= n.
 *   (k <= 8192 runs a persistent kernel that keeps the activation in registers; longer k
 *   a per-strip kernel that reads it from L2.  Both sum in a fixed order per k.)
 * Errors: FP8Q_EINVAL, FP8Q_ENULL, FP8Q_EALIGN, FP8Q_ELAUNCH. */
int w8a16_block_gemv(const uint16_t* a, const uint8_t* w_q, const float* w_scale,
                     uint16_t* out, int32_t m, int32_t n, int32_t k, int32_t ldc,
                     hipStream_t stream);

/* Several projections of one bf16 activation in one launch (as w8a8_block_gemm_grouped):
 * each projs[p] gets exactly what w8a16_block_gemv computes for it. 1 <= count <= 8. */
int w8a16_block_gemv_grouped(const uint16_t* a, const fp8q_gemm_proj* projs, int32_t count,
                             int32_t m, int32_t k, hipStream_t stream);

/* --------------------------------------------------------- paged FP8 KV write
 * [staging] Fp8KvWriteTarget and replay_and_release (the write's arguments: strides in
 * elements, pool stride = block_size * heads * head_dim); [staging] module doc: one scale
 * per tensor, later writes of a slot replace earlier ones.
 *
 * For each token t < num_tokens with 0 <= slot < num_blocks * block_size (slot =
 * slot_mapping[t]; other slots are skipped -- negative ones are padding):
 *   b = slot / block_size, o = slot % block_size, for all h < H, d < D:
 *   k_cache[b * cache_stride + (o * H + h) * D + d] = E4M3(k[t * key_stride + h*D + d] / k_scale)
 *   v_cache[... same index ...]                       = E4M3(v[t * value_stride + h*D + d] / v_scale)
 * Slots must be distinct within one call (two tokens on one slot race).
 *
 *   k, v            device bf16 rows of key_stride / value_stride elements
 *   k_cache,v_cache device uint8 pools of num_blocks * cache_stride bytes each
 *   slot_mapping    device int64 [num_tokens]
 *   num_tokens >= 0 (0 is a no-op); num_kv_heads, head_dim, block_size, num_blocks > 0;
 *   key_stride, value_stride >= H*D; cache_stride >= block_size*H*D;
 *   k_scale, v_scale in [2^-64, 2^64] (dequantization multipliers).
 * The vector path needs 16-byte aligned k/v/pools and H*D, strides, cache_stride all
 * multiples of 8; anything else takes an element-wise path with the same results.
 * Errors: FP8Q_EINVAL, FP8Q_ENULL, FP8Q_ELAUNCH. */
int fp8_kv_write(const uint16_t* k, const uint16_t* v, uint8_t* k_cache, uint8_t* v_cache,
                 const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                 int32_t head_dim, int32_t block_size, int64_t num_blocks, float k_scale,
                 float v_scale, int32_t key_stride, int32_t value_stride,
                 int64_t cache_stride, hipStream_t stream);

/* [calib] Fp8KvCalibration::observe + [staging] module doc, in one pass: inside the
 * calibration window every batch is both measured (absmax) and written (at the provisional
 * scale).  Exactly fp8_kv_write(...) followed by fp8_kv_amax over the same batch's rows:
 *   amax2[0] = max(amax2[0], max |k[t * key_stride + i]|), amax2[1] likewise for v, over
 *   every t < num_tokens and i < H*D (padding tokens included: the batch's data, as the
 *   pages' absmax), with the pools written as fp8_kv_write writes them.
 * One kernel when H*D is a multiple of 16 up to 512 and the rows are 16-byte aligned; else
 * the absmax pass and the write run back to back.  amax2: device fp32[2], 4-byte aligned.
 * Errors as fp8_kv_write, and FP8Q_ENULL for a NULL amax2. */
int fp8_kv_write_amax(const uint16_t* k, const uint16_t* v, uint8_t* k_cache,
                      uint8_t* v_cache, const int64_t* slot_mapping, int32_t num_tokens,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int64_t num_blocks, float k_scale, float v_scale, int32_t key_stride,
                      int32_t value_stride, int64_t cache_stride, float* amax2,
                      hipStream_t stream);

/* ------------------------------------------------------ paged FP8 KV read (dequant)
 * [staging] module doc: every token of a sequence's history is read back at the one
 * per-tensor scale the layer holds (which is why early tokens written at the provisional
 * scale must be rewritten at the frozen one); the write above defines the pool layout.
 *
 * For each token t < num_tokens with 0 <= slot < num_blocks * block_size (slot =
 * slot_mapping[t]; output rows of other tokens are left untouched):
 *   b = slot / block_size, o = slot % block_size, for all h < H, d < D:
 *   k_out[t * out_key_stride + h*D + d] =
 *       bf16_rne(fp32(E4M3 value of k_cache[b * cache_stride + (o * H + h) * D + d]) * k_scale)
 *   v_out[... same ...] likewise with v_cache and v_scale
 * The product is one binary32 multiplication (round to nearest even), then rounded to
 * bf16 to nearest even; the NaN codes 0x7F / 0xFF read as the quiet NaN 0x7FC0.
 *
 *   k_cache, v_cache   device uint8 pools of num_blocks * cache_stride bytes each
 *   slot_mapping       device int64 [num_tokens]
 *   k_out, v_out       device bf16 rows of out_key_stride / out_value_stride elements
 *   num_tokens >= 0 (0 is a no-op); num_kv_heads, head_dim, block_size, num_blocks > 0;
 *   out strides >= H*D; cache_stride >= block_size*H*D; scales in [2^-64, 2^64].
 * The vector path needs H*D, the output strides and cache_stride multiples of 8, 8-byte
 * aligned pools and 16-byte aligned outputs; anything else takes an element-wise path
 * with the same results.
 * Errors: FP8Q_EINVAL, FP8Q_ENULL, FP8Q_EALIGN, FP8Q_ELAUNCH. */
int fp8_kv_read(const uint8_t* k_cache, const uint8_t* v_cache, const int64_t* slot_mapping,
                int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                int64_t num_blocks, float k_scale, float v_scale, uint16_t* k_out,
                uint16_t* v_out, int32_t out_key_stride, int32_t out_value_stride,
                int64_t cache_stride, hipStream_t stream);

/* ------------------------------------------------------------- KV absolute max
 * [calib] Fp8KvCalibration::absmax: max |K| and max |V| of a batch, max-accumulated into
 * a device float[2] that the caller zeroes once (so a window's running max can stay on
 * the device).
 *   amax2[0] = max(amax2[0], max_i |k[i]|), amax2[1] = max(amax2[1], max_i |v[i]|)
 *   k, v device bf16 [n_elems] packed; amax2 device fp32[2], 4-byte aligned, >= +0.0
 *   n_elems >= 0.  Errors: FP8Q_EINVAL, FP8Q_ENULL, FP8Q_ELAUNCH. */
int fp8_kv_amax(const uint16_t* k, const uint16_t* v, int64_t n_elems, float* amax2,
                hipStream_t stream);

/* ----------------------------------------------- online KV scale calibrator
 * [calib] module doc, PROVISIONAL_SCALE, Fp8KvCalibration::{new, observe, scales};
 * [staging] module doc ("The fix, and its tradeoff"), KvStaging::{stage,
 * replay_and_release, release}, MAX_STAGED_TOKENS.
 *
 * One attention layer's per-tensor K/V scale calibration.  Inside the window each
 * observed batch's |K|/|V| maximum folds into a running maximum kept on the device, and
 * the batch (bf16 rows + slots) is copied into packed staging; the caller then writes
 * it at the provisional scale.  The observe whose token count reaches the window freezes
 * scale = (max(amax, 1e-10) * headroom) / 448 for K and V over every observed token
 * including its own batch, replays the staged batches at the frozen scales into the
 * target pools (one write of every staged token whose slot no later staged token writes,
 * which leaves the bytes an in-order replay leaves), and releases the staging in stream
 * order; the caller then writes that batch at the frozen scales.  Later observes do
 * nothing.  A batch whose heads x head_dim differ from the first staged batch, or that
 * would overflow the window's staging, is not staged (it keeps the provisional scale).
 * The window is clamped to 4096 tokens and headroom to >= 1.
 * Call order per batch: fp8q_kv_calib_observe, then fp8q_kv_calib_scales, then the
 * caller's fp8_kv_write of that batch, all on one stream.  Not capturable in a HIP graph
 * (the freeze reads the running maximum back to the host). */
typedef struct fp8q_kv_calib fp8q_kv_calib;

/* Where the replay writes (the live write's own pools and geometry). */
typedef struct fp8q_kv_target {
  uint8_t* k_pool;
  uint8_t* v_pool;
  const int64_t* slot_mapping; /* this batch's slots, int64 [num_tokens] */
  int32_t block_size;
  int32_t key_stride;          /* row stride of the observed K, elements */
  int32_t value_stride;        /* row stride of the observed V, elements */
  int32_t reserved;
  int64_t cache_stride;        /* elements per block = block_size * H * D or more */
  int64_t num_blocks;          /* blocks in each pool */
} fp8q_kv_target;

typedef struct fp8q_kv_calib_info {
  int32_t window_tokens;    /* after the 4096 clamp */
  int32_t requested_tokens; /* as passed to create */
  int32_t frozen;
  int32_t staged_batches;
  int64_t tokens_seen;
  int64_t staged_tokens;
  int64_t unstaged_tokens;  /* tokens of declined batches */
  int64_t replayed_tokens;  /* tokens rewritten at the freeze */
  float k_scale;            /* provisional until frozen */
  float v_scale;
  float k_amax;             /* running maxima read at the freeze (0 before) */
  float v_amax;
  float headroom;           /* after the >= 1 clamp */
  float provisional_scale;
} fp8q_kv_calib_info;

/* What observe would do with a batch, without doing it. */
#define FP8Q_CALIB_STAGE 0
#define FP8Q_CALIB_DECLINE 1
#define FP8Q_CALIB_FREEZE 2
#define FP8Q_CALIB_FROZEN 3

/* The device work of a calibrator, as a table of callbacks ([staging] and [calib] take a
 * GPU backend object for the same purpose).  The calibrator's bookkeeping (window, stage,
 * decline, freeze formula and range check, replay order, counters) only calls these; it
 * never touches device memory itself, so a table backed by host memory runs the whole
 * state machine on a CPU.  fp8q_kv_calib_create uses the library's own HIP table.
 * Every callback returns FP8Q_OK or a negative FP8Q_E* status, which observe returns.
 *   device      the current device (observe refuses a device other than the first one)
 *   alloc       *out = `bytes` of device memory, usable by work enqueued on `stream` after
 *               this call (HIP: hipMallocAsync)
 *   release     free what alloc returned: in stream order after the work enqueued on
 *               `stream` when at_destroy == 0; when at_destroy != 0 (from
 *               fp8q_kv_calib_destroy, stream unused) only once all device work is done
 *   zero        bytes of p = 0, stream-ordered
 *   amax_rows   amax2[0] = max(amax2[0], max|k|), amax2[1] likewise for v, over `rows` rows of
 *               `elems` bf16 at key/value strides (elements), stream-ordered
 *   copy2d      `rows` rows of row_bytes bytes from src (rows src_pitch bytes apart) to dst,
 *               packed, stream-ordered
 *   read        bytes from device src to host dst once the work enqueued on `stream` is done
 *               (blocks the caller)
 *   replay      write n staged packed rows (`elems` bf16 each, K and V) to the target's pools
 *               at (k_scale, v_scale) as fp8_kv_write would write them one after another in
 *               staging order (a slot staged twice keeps its later row); scratch_slots is
 *               int64 [n] of device scratch the callback may use; stream-ordered
 *   stage       optional (NULL: amax_rows, then copy2d of the K rows, V rows and slots): the
 *               same in one call -- amax_rows over the batch, its rows copied packed to
 *               dst_k / dst_v (row t at t * elems) and its `rows` slots to dst_slots */
typedef struct fp8q_kv_calib_ops {
  void* ctx;
  int (*device)(void* ctx, int32_t* dev);
  int (*alloc)(void* ctx, uint64_t bytes, void** out, hipStream_t stream);
  int (*release)(void* ctx, void* p, hipStream_t stream, int32_t at_destroy);
  int (*zero)(void* ctx, void* p, uint64_t bytes, hipStream_t stream);
  int (*amax_rows)(void* ctx, const uint16_t* k, const uint16_t* v, int64_t rows,
                   int64_t elems, int64_t key_stride, int64_t value_stride, float* amax2,
                   hipStream_t stream);
  int (*copy2d)(void* ctx, void* dst, const void* src, int64_t src_pitch, int64_t row_bytes,
                int64_t rows, hipStream_t stream);
  int (*read)(void* ctx, void* host_dst, const void* src, uint64_t bytes, hipStream_t stream);
  int (*replay)(void* ctx, const uint16_t* k, const uint16_t* v, const int64_t* slots,
                int64_t* scratch_slots, int32_t n, int32_t elems, const fp8q_kv_target* target,
                float k_scale, float v_scale, hipStream_t stream);
  int (*stage)(void* ctx, const uint16_t* k, const uint16_t* v, const int64_t* slots,
               int64_t rows, int64_t elems, int64_t key_stride, int64_t value_stride,
               uint16_t* dst_k, uint16_t* dst_v, int64_t* dst_slots, float* amax2,
               hipStream_t stream);
} fp8q_kv_calib_ops;

/* window_tokens > 0 (window 0 means no calibrator: FP8Q_EINVAL); headroom finite and
 * <= 2^64 (values below 1 are raised to 1); provisional_scale in [2^-64, 2^64] (the
 * pages use 2.0).  Allocates host state only; device buffers are allocated on the first
 * observe, on the device current then.  *out receives the handle.
 * Errors: FP8Q_EINVAL, FP8Q_ENULL, FP8Q_EHIP (host allocation). */
int fp8q_kv_calib_create(int32_t window_tokens, float headroom, float provisional_scale,
                         fp8q_kv_calib** out);
/* As fp8q_kv_calib_create, with the device work going through `ops` (copied; every
 * callback but stage must be set; the table's ctx must outlive the calibrator). */
int fp8q_kv_calib_create_with_ops(int32_t window_tokens, float headroom,
                                  float provisional_scale, const fp8q_kv_calib_ops* ops,
                                  fp8q_kv_calib** out);
/* Fold one batch in (see above).  k, v: device bf16 [num_tokens] rows at the target's
 * key/value strides.  Enqueues work on `stream`; blocks only at the freeze, to read the
 * 8-byte running maximum back (through 64 bytes of page-locked host memory that the first
 * freeze of the process allocates and every later one reuses; concurrent freezes take
 * turns).  The first staged batch allocates the staging in one piece
 * (window * H * D * 2 * 2 + window * 16 bytes, stream-ordered); the freeze releases it in
 * stream order.  With the library's HIP table an in-window observe is one kernel (absmax
 * and staging copy in one pass).
 * A frozen scale outside [2^-64, 2^64] (the write's scale range) fails the freezing
 * observe with FP8Q_EINVAL and leaves the calibrator as it was (the batch's absmax may
 * already be folded into the running maximum; folding the same batch again changes
 * nothing).
 * Errors: FP8Q_EINVAL, FP8Q_ENULL, FP8Q_EHIP, FP8Q_ELAUNCH, FP8Q_ESTATE. */
int fp8q_kv_calib_observe(fp8q_kv_calib* c, const uint16_t* k, const uint16_t* v,
                          int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                          const fp8q_kv_target* target, hipStream_t stream);
/* Pure query: FP8Q_CALIB_* for a batch of num_tokens x elems_per_token, or < 0. */
int fp8q_kv_calib_decide(const fp8q_kv_calib* c, int32_t num_tokens,
                         int32_t elems_per_token);
/* The scales the caller writes with now (provisional until the freeze). */
int fp8q_kv_calib_scales(const fp8q_kv_calib* c, float* k_scale, float* v_scale);
/* Snapshot of the calibrator's counters, scales and running maxima. */
int fp8q_kv_calib_state(const fp8q_kv_calib* c, fp8q_kv_calib_info* info);
/* Frees staging and device state (after all device work is done). NULL ok. */
void fp8q_kv_calib_destroy(fp8q_kv_calib* c);

#ifdef __cplusplus
}
#endif

#endif /* FP8Q_H */
