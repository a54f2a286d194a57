/*
 * fp8_oracle.c -- plain, slow, obviously-correct CPU oracle for the FP8 (OCP E4M3)
 * quantize-and-consume path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call this file: only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg load it.  It shares
 * no code, header, table or constant generator with the HIP library.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -shared -fPIC (see oracle/build.py).
 * -ffp-contract=off keeps every a*b+c as two IEEE roundings; x86-64 SSE evaluates float
 * expressions in float (FLT_EVAL_METHOD == 0), so "float / float" is one correctly
 * rounded IEEE binary32 division.
 *
 * Sources (pages as published; cited by page title and the item on the page):
 *  [calib]   metrale_model_layers/layers/fp8_calibration.rs -- module doc (window, freeze
 *            formula amax*headroom/448, invariants), PROVISIONAL_SCALE, Fp8KvCalibration::new
 *            (headroom and window clamps), ::observe (stage / freeze / frozen), ::absmax.
 *  [staging] spark_model/layers/fp8_calibration/staging.rs -- module doc "The fix, and its
 *            tradeoff" (chronological replay, last writer wins, crossing batch written after
 *            the replay, staging cost), MAX_STAGED_TOKENS, Fp8KvWriteTarget (strides, pool
 *            stride), KvStaging::stage (lazy allocation, decline), ::replay_and_release.
 *  [actq]    spark_model/layers/ops/fp8_act_quant.rs -- module doc (1x128 K-groups, one group
 *            per token row and K-group; variants must emit identical bytes).
 *  [decode]  spark_model/layers/ops/dispatch_proj_decode.rs -- module doc "NUMERICS" (E4M3
 *            activations with per-token 1x128 FP32 scales, 128x128 FP32 weight block scales,
 *            FP32 epilogue; 3 stored mantissa bits), DecodeW8a8Plan / decode_w8a8_selected
 *            (scale grid [N/128, K/128], activation scales [M, K/128]), decode_w8a8_gemm.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - E4M3 is the OCP "FN" encoding: bias 7, no infinities, S.1111.111 is NaN, 448 max.
 *  - fp32 -> E4M3 is round-to-nearest-even with saturation to +-448 (the pages say values
 *    out of range are clipped, never NaN); the sign is kept, so a negative value that
 *    rounds to zero encodes as 0x80.
 *  - A value is divided by its scale (IEEE fp32 division), then encoded.
 *  - The scale of an all-zero group is floored: s = max(amax, 1e-10f) / 448.
 *  - Inputs are finite; NaN/Inf inputs are outside the contract (asserted here).
 */
#include <assert.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_E4M3_MAX 448.0
#define ORACLE_AMAX_FLOOR 1e-10f

/* ------------------------------------------------------------------ bf16 / f32 bits */

static float f32_from_bits(uint32_t b) {
  float f;
  memcpy(&f, &b, 4);
  return f;
}

static uint32_t f32_bits(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  return b;
}

/* bfloat16 is the top half of an IEEE binary32: widening is exact. */
float oracle_bf16_to_f32(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/* ------------------------------------------------------------------ C1: E4M3 decode */

/* Value of an OCP E4M3 code, exactly, as a double.  Bit layout S EEEE MMM, bias 7.
 * E == 0: subnormal, M * 2^-9.  E == 15 and M == 7: NaN.  Otherwise (1 + M/8) * 2^(E-7). */
double oracle_e4m3_decode(uint8_t code) {
  int s = code >> 7;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* ------------------------------------------- C2 (i): E4M3 encode by fp32 bit surgery */

/* Round |v| to E4M3 with round-to-nearest-even, saturating at 448.  Works on the binary32
 * fields directly: the normal E4M3 range keeps the top 3 of the 23 stored mantissa bits,
 * the subnormal range is an integer multiple of 2^-9. */
uint8_t oracle_e4m3_encode_bits(float v) {
  uint32_t b = f32_bits(v);
  uint8_t sign = (uint8_t)((b >> 31) << 7);
  uint32_t a = b & 0x7FFFFFFFu;
  uint32_t e = a >> 23; /* biased binary32 exponent */
  assert(e != 0xFF && "non-finite input is outside the contract");
  if (a >= 0x43E00000u) /* |v| >= 448: clip to the largest finite code */
    return sign | 0x7E;
  if (e >= 121) { /* |v| >= 2^-6: normal E4M3, E = e - 120 */
    uint32_t t = a >> 20;   /* exponent and the top 3 mantissa bits */
    uint32_t rem = a & 0xFFFFF; /* the 20 discarded bits */
    if (rem > 0x80000u || (rem == 0x80000u && (t & 1u))) t += 1; /* carry may bump E */
    return sign | (uint8_t)(t - (120u << 3));
  }
  /* |v| < 2^-6: code = RNE(|v| * 2^9), an integer 0..8 (8 is the smallest normal). */
  {
    uint32_t mant = (e == 0) ? (a & 0x7FFFFF) : ((a & 0x7FFFFF) | 0x800000);
    int eu = (e == 0) ? 1 : (int)e; /* subnormal binary32 shares exponent 1's scale */
    /* |v| = mant * 2^(eu - 150);  |v| * 2^9 = mant * 2^(eu - 141) = mant >> (141 - eu). */
    int shift = 141 - eu; /* >= 21 here */
    uint32_t q, r, half;
    if (shift >= 32) return sign; /* mant < 2^24 <= 2^(shift-8): far below one half */
    q = mant >> shift;
    r = mant & ((1u << shift) - 1u);
    half = 1u << (shift - 1);
    if (r > half || (r == half && (q & 1u))) q += 1;
    return sign | (uint8_t)q;
  }
}

/* --------------------------------- C2 (ii): E4M3 encode by search of the decode table */

/* Largest finite non-negative codes 0x00..0x7E decoded once; strictly increasing. */
static double g_pos[127];
static int g_pos_ready = 0;

static void oracle_init_table(void) {
  int c;
  if (g_pos_ready) return;
  for (c = 0; c <= 0x7E; ++c) g_pos[c] = oracle_e4m3_decode((uint8_t)c);
  g_pos_ready = 1;
}

/* Nearest E4M3 value by binary search over the 127 non-negative finite values; a value
 * exactly half-way between two neighbours takes the even code (mantissa LSB 0);
 * anything at or above 448 takes 448.  All comparisons are exact in double. */
uint8_t oracle_e4m3_encode_search(float v) {
  double x = (double)v;
  uint8_t sign = (uint8_t)((f32_bits(v) >> 31) << 7);
  double ax = fabs(x);
  int lo = 0, hi = 0x7E, c;
  double mid;
  assert(isfinite(x) && "non-finite input is outside the contract");
  oracle_init_table();
  if (ax >= ORACLE_E4M3_MAX) return sign | 0x7E;
  /* invariant: g_pos[lo] <= ax < g_pos[hi] */
  while (hi - lo > 1) {
    int m = (lo + hi) / 2;
    if (g_pos[m] <= ax)
      lo = m;
    else
      hi = m;
  }
  if (g_pos[lo] == ax) return sign | (uint8_t)lo;
  mid = 0.5 * (g_pos[lo] + g_pos[hi]); /* exact: both are short dyadic numbers */
  if (ax < mid)
    c = lo;
  else if (ax > mid)
    c = hi;
  else
    c = (lo % 2 == 0) ? lo : hi;
  return sign | (uint8_t)c;
}

/* Batch forms for the self-tests (exhaustive sweeps stay in C for speed). */
void oracle_e4m3_encode_bits_n(const float* v, uint8_t* out, int64_t n) {
  int64_t i;
  for (i = 0; i < n; ++i) out[i] = oracle_e4m3_encode_bits(v[i]);
}

void oracle_e4m3_encode_search_n(const float* v, uint8_t* out, int64_t n) {
  int64_t i;
  for (i = 0; i < n; ++i) out[i] = oracle_e4m3_encode_search(v[i]);
}

/* Count disagreements between (i) and (ii) over every binary32 bit pattern in
 * [lo_bits, hi_bits] (inclusive, positive patterns), both signs.  Returns the number of
 * mismatches and the first mismatching pattern in *first (or 0xFFFFFFFF). */
int64_t oracle_e4m3_sweep_compare(uint32_t lo_bits, uint32_t hi_bits, uint32_t* first) {
  int64_t bad = 0;
  uint64_t b;
  *first = 0xFFFFFFFFu;
  oracle_init_table();
  for (b = lo_bits; b <= hi_bits; ++b) {
    float p = f32_from_bits((uint32_t)b);
    float n = f32_from_bits((uint32_t)b | 0x80000000u);
    if (oracle_e4m3_encode_bits(p) != oracle_e4m3_encode_search(p) ||
        oracle_e4m3_encode_bits(n) != oracle_e4m3_encode_search(n)) {
      if (bad == 0) *first = (uint32_t)b;
      ++bad;
    }
  }
  return bad;
}

/* --------------------------------------------- C3: per-token 1x128 group quantization */

/* x: bf16 [m, k] row-major; q: E4M3 [m, k]; scales: fp32 [m, k/128] token-major.
 * For every row and 128-wide K-group: amax = max |x| (exact), s = max(amax, 1e-10f)/448
 * (one fp32 division), code = E4M3(fp32(x) / s). */
void oracle_group_quant(const uint16_t* x, int64_t m, int64_t k, uint8_t* q,
                        float* scales) {
  int64_t r, g, j, groups = k / 128;
  assert(k % 128 == 0);
  for (r = 0; r < m; ++r) {
    for (g = 0; g < groups; ++g) {
      const uint16_t* xg = x + r * k + g * 128;
      float amax = 0.0f, s;
      for (j = 0; j < 128; ++j) {
        float a = fabsf(oracle_bf16_to_f32(xg[j]));
        assert(isfinite(a));
        if (a > amax) amax = a;
      }
      s = (amax > ORACLE_AMAX_FLOOR ? amax : ORACLE_AMAX_FLOOR) / 448.0f;
      scales[r * groups + g] = s;
      for (j = 0; j < 128; ++j) {
        float qv = oracle_bf16_to_f32(xg[j]) / s;
        q[r * k + g * 128 + j] = oracle_e4m3_encode_bits(qv);
      }
    }
  }
}

/* ---------------------------------------------- C4: 128x128 weight block quantization */

/* w: bf16 [n, k] row-major; wq: E4M3 [n, k]; ws: fp32 [ceil(n/128), ceil(k/128)] with
 * block (nb, kb) at nb * ceil(k/128) + kb.  Same formula as C3, over a 128x128 block
 * (blocks at the right/bottom edge are clipped to the matrix). */
void oracle_block_quant(const uint16_t* w, int64_t n, int64_t k, uint8_t* wq, float* ws) {
  int64_t nbs = (n + 127) / 128, kbs = (k + 127) / 128, nb, kb, i, j;
  for (nb = 0; nb < nbs; ++nb) {
    for (kb = 0; kb < kbs; ++kb) {
      int64_t i1 = (nb + 1) * 128 < n ? (nb + 1) * 128 : n;
      int64_t j1 = (kb + 1) * 128 < k ? (kb + 1) * 128 : k;
      float amax = 0.0f, s;
      for (i = nb * 128; i < i1; ++i)
        for (j = kb * 128; j < j1; ++j) {
          float a = fabsf(oracle_bf16_to_f32(w[i * k + j]));
          assert(isfinite(a));
          if (a > amax) amax = a;
        }
      s = (amax > ORACLE_AMAX_FLOOR ? amax : ORACLE_AMAX_FLOOR) / 448.0f;
      ws[nb * kbs + kb] = s;
      for (i = nb * 128; i < i1; ++i)
        for (j = kb * 128; j < j1; ++j)
          wq[i * k + j] = oracle_e4m3_encode_bits(oracle_bf16_to_f32(w[i * k + j]) / s);
    }
  }
}

/* ------------------------------------------------------ C5: block-scaled W8A8 GEMM */

/* ref[m, n] = sum_k (dec(a_q[m,k]) * a_s[m, k/128]) * (dec(w_q[n,k]) * w_s[n/128, k/128]),
 * every product and sum in double, plain triple loop, in K order.
 * a_q [m, k], a_s [m, k/128], w_q [n, k] (K contiguous), w_s [ceil(n/128), k/128]. */
void oracle_gemm(const uint8_t* a_q, const float* a_s, const uint8_t* w_q, const float* w_s,
                 int64_t m, int64_t n, int64_t k, double* ref) {
  int64_t i, j, kk, groups = k / 128;
  double dec[256];
  for (i = 0; i < 256; ++i) dec[i] = oracle_e4m3_decode((uint8_t)i);
  assert(k % 128 == 0);
  for (i = 0; i < m; ++i) {
    for (j = 0; j < n; ++j) {
      double acc = 0.0;
      for (kk = 0; kk < k; ++kk) {
        double a = dec[a_q[i * k + kk]] * (double)a_s[i * groups + kk / 128];
        double w = dec[w_q[j * k + kk]] * (double)w_s[(j / 128) * groups + kk / 128];
        acc += a * w;
      }
      ref[i * n + j] = acc;
    }
  }
}

/* -------------------------------------------- W8A16: bf16 activation x E4M3 weight */

/* The decode page's small-batch tier (module doc, NUMERICS; DECODE_W8A8_ROWS): the
 * activation stays bf16 and multiplies E4M3 weights carrying the same 128x128 FP32 block
 * scales.  ref[m, n] = sum_k bf16(a[m,k]) * dec(w_q[n,k]) * w_s[n/128, k/128] and
 * absref[m, n] = sum_k |same term|, every product and sum in double, K order (each term is
 * exact in double: 8 + 4 + 24 significant bits). */
void oracle_gemm_w8a16(const uint16_t* a, const uint8_t* w_q, const float* w_s, int64_t m,
                       int64_t n, int64_t k, double* ref, double* absref) {
  int64_t i, j, kk, groups = k / 128;
  double dec[256];
  for (i = 0; i < 256; ++i) dec[i] = oracle_e4m3_decode((uint8_t)i);
  assert(k % 128 == 0);
  for (i = 0; i < m; ++i) {
    for (j = 0; j < n; ++j) {
      double acc = 0.0, mag = 0.0;
      for (kk = 0; kk < k; ++kk) {
        double t = (double)oracle_bf16_to_f32(a[i * k + kk]) * dec[w_q[j * k + kk]] *
                   (double)w_s[(j / 128) * groups + kk / 128];
        acc += t;
        mag += fabs(t);
      }
      ref[i * n + j] = acc;
      absref[i * n + j] = mag;
    }
  }
}

/* -------------------------------------------------------------- C7: absolute max */

/* max |x| over n bf16 values, max-accumulated into *acc (the caller zeroes it). */
void oracle_amax(const uint16_t* x, int64_t n, float* acc) {
  int64_t i;
  float a = *acc;
  for (i = 0; i < n; ++i) {
    float v = fabsf(oracle_bf16_to_f32(x[i]));
    assert(isfinite(v));
    if (v > a) a = v;
  }
  *acc = a;
}

/* ------------------------------------------------------------- C6: paged KV write */

/* For tokens t = 0..T-1 in order: a negative slot is skipped; otherwise block b =
 * slot / block_size, offset o = slot % block_size and, for every head h and dim d,
 *   kc[b*cs + (o*H + h)*D + d] = E4M3(fp32(K[t*ks + h*D + d]) / k_scale)
 * and the same for V.  Later tokens overwrite earlier ones on a repeated slot. */
void oracle_kv_write(const uint16_t* kx, const uint16_t* vx, uint8_t* kc, uint8_t* vc,
                     const int64_t* slots, int64_t T, int64_t H, int64_t D,
                     int64_t block_size, float k_scale, float v_scale, int64_t ks,
                     int64_t vs, int64_t cs) {
  int64_t t, h, d;
  for (t = 0; t < T; ++t) {
    int64_t slot = slots[t], b, o;
    if (slot < 0) continue;
    b = slot / block_size;
    o = slot % block_size;
    for (h = 0; h < H; ++h)
      for (d = 0; d < D; ++d) {
        int64_t dst = b * cs + (o * H + h) * D + d;
        kc[dst] = oracle_e4m3_encode_bits(oracle_bf16_to_f32(kx[t * ks + h * D + d]) / k_scale);
        vc[dst] = oracle_e4m3_encode_bits(oracle_bf16_to_f32(vx[t * vs + h * D + d]) / v_scale);
      }
  }
}

/* ------------------------------------------------------ paged KV read (dequantize) */

/* bf16 bit pattern of a binary32, round to nearest even; every NaN maps to the one quiet
 * NaN 0x7FC0 (the pages never store a NaN code, so its read-back is only required to be a
 * NaN; one fixed pattern keeps the result byte-comparable). */
static uint16_t oracle_f32_to_bf16(float f) {
  uint32_t b = f32_bits(f);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

/* Attention-side read of a paged history at one scale (staging module doc: a sequence's
 * history is dequantized with one k_scale / v_scale): for each token with a slot in
 * [0, num_blocks * block_size), every element is bf16(fp32(dec(code)) * scale), the
 * product one binary32 multiplication rounded to nearest even, then rounded to bf16.
 * Tokens with other slots are left untouched. */
void oracle_kv_read(const uint8_t* kc, const uint8_t* vc, const int64_t* slots, int64_t T,
                    int64_t H, int64_t D, int64_t block_size, int64_t num_blocks,
                    float k_scale, float v_scale, uint16_t* ko, uint16_t* vo, int64_t ks,
                    int64_t vs, int64_t cs) {
  int64_t t, h, d;
  for (t = 0; t < T; ++t) {
    int64_t slot = slots[t], b, o;
    if (slot < 0 || slot >= num_blocks * block_size) continue;
    b = slot / block_size;
    o = slot % block_size;
    for (h = 0; h < H; ++h)
      for (d = 0; d < D; ++d) {
        int64_t src = b * cs + (o * H + h) * D + d;
        float kd = (float)oracle_e4m3_decode(kc[src]);
        float vd = (float)oracle_e4m3_decode(vc[src]);
        ko[t * ks + h * D + d] = oracle_f32_to_bf16(kd * k_scale);
        vo[t * vs + h * D + d] = oracle_f32_to_bf16(vd * v_scale);
      }
  }
}

/* ------------------------------------------------ C8: online KV scale calibration */

/* One layer's calibrator, modelled step by step from [calib] and [staging]:
 *  - window W = min(window, 4096), headroom h = max(headroom, 1), provisional p = 2.0;
 *  - inside the window each batch's |K|/|V| max folds into the running max and the token
 *    count; if the count has not reached W the batch is staged (packed bf16 copy + slots)
 *    and written at p; a batch whose elements-per-token differ from the first staged
 *    batch, or that would overflow W staged tokens, is declined and stays at p;
 *  - the batch whose count reaches W freezes scale = (max(amax,1e-10)*h)/448 for K and V,
 *    replays every staged batch in order at the frozen scales, drops the staging, and is
 *    then written by the caller at the frozen scales (it is never staged);
 *  - once frozen, writes use the frozen scales. */
typedef struct {
  int64_t window, tokens_seen, staged_tokens, staged_batches, unstaged_tokens;
  int64_t replayed_tokens, elems_per_token, capacity;
  float headroom, provisional, k_scale, v_scale, k_max, v_max;
  int frozen;
  /* staging (host copies) */
  uint16_t *sk, *sv;
  int64_t* sslots;
  int64_t* batch_off;
  int64_t* batch_n;
} oracle_calib;

oracle_calib* oracle_calib_create(int64_t window, float headroom, float provisional) {
  oracle_calib* c = (oracle_calib*)calloc(1, sizeof(oracle_calib));
  c->window = window < 4096 ? window : 4096;
  c->headroom = headroom >= 1.0f ? headroom : 1.0f;
  c->provisional = provisional;
  c->k_scale = provisional;
  c->v_scale = provisional;
  return c;
}

void oracle_calib_destroy(oracle_calib* c) {
  if (!c) return;
  free(c->sk);
  free(c->sv);
  free(c->sslots);
  free(c->batch_off);
  free(c->batch_n);
  free(c);
}

/* Observe one packed batch (K and V [T, H*D] bf16, slots [T]) and then perform the
 * caller's own write of that batch at the scales in force afterwards.  Returns the step
 * taken: 0 = staged, 1 = declined (kept at provisional), 2 = froze, 3 = already frozen. */
int oracle_calib_observe_and_write(oracle_calib* c, const uint16_t* kx, const uint16_t* vx,
                                   const int64_t* slots, int64_t T, int64_t H, int64_t D,
                                   int64_t block_size, int64_t cs, uint8_t* kc,
                                   uint8_t* vc) {
  int64_t e = H * D;
  int step;
  if (c->frozen) {
    step = 3;
  } else {
    float km = 0.0f, vm = 0.0f;
    oracle_amax(kx, T * e, &km);
    oracle_amax(vx, T * e, &vm);
    if (km > c->k_max) c->k_max = km;
    if (vm > c->v_max) c->v_max = vm;
    c->tokens_seen += T;
    if (c->tokens_seen >= c->window) {
      int64_t b;
      float kfl = c->k_max > ORACLE_AMAX_FLOOR ? c->k_max : ORACLE_AMAX_FLOOR;
      float vfl = c->v_max > ORACLE_AMAX_FLOOR ? c->v_max : ORACLE_AMAX_FLOOR;
      c->k_scale = (kfl * c->headroom) / 448.0f;
      c->v_scale = (vfl * c->headroom) / 448.0f;
      for (b = 0; b < c->staged_batches; ++b) {
        int64_t off = c->batch_off[b];
        oracle_kv_write(c->sk + off * c->elems_per_token, c->sv + off * c->elems_per_token,
                        kc, vc, c->sslots + off, c->batch_n[b], H, D, block_size,
                        c->k_scale, c->v_scale, c->elems_per_token, c->elems_per_token, cs);
      }
      c->replayed_tokens = c->staged_tokens;
      c->frozen = 1;
      step = 2;
    } else {
      if (c->capacity == 0) { /* lazy allocation at the first staged batch */
        c->capacity = c->window;
        c->elems_per_token = e;
        c->sk = (uint16_t*)malloc((size_t)(c->capacity * e) * 2);
        c->sv = (uint16_t*)malloc((size_t)(c->capacity * e) * 2);
        c->sslots = (int64_t*)malloc((size_t)c->capacity * 8);
        c->batch_off = (int64_t*)malloc((size_t)c->capacity * 8);
        c->batch_n = (int64_t*)malloc((size_t)c->capacity * 8);
      }
      if (e != c->elems_per_token || c->staged_tokens + T > c->capacity) {
        c->unstaged_tokens += T;
        step = 1;
      } else {
        memcpy(c->sk + c->staged_tokens * e, kx, (size_t)(T * e) * 2);
        memcpy(c->sv + c->staged_tokens * e, vx, (size_t)(T * e) * 2);
        memcpy(c->sslots + c->staged_tokens, slots, (size_t)T * 8);
        c->batch_off[c->staged_batches] = c->staged_tokens;
        c->batch_n[c->staged_batches] = T;
        c->staged_batches += 1;
        c->staged_tokens += T;
        step = 0;
      }
    }
  }
  /* the caller's write of this batch, at the scales now in force */
  oracle_kv_write(kx, vx, kc, vc, slots, T, H, D, block_size, c->k_scale, c->v_scale, e, e,
                  cs);
  return step;
}

/* Snapshot of the calibrator's counters and scales. */
void oracle_calib_info(const oracle_calib* c, int64_t* counters, float* values) {
  counters[0] = c->window;
  counters[1] = c->tokens_seen;
  counters[2] = c->staged_tokens;
  counters[3] = c->staged_batches;
  counters[4] = c->unstaged_tokens;
  counters[5] = c->replayed_tokens;
  counters[6] = c->frozen;
  values[0] = c->k_scale;
  values[1] = c->v_scale;
  values[2] = c->k_max;
  values[3] = c->v_max;
  values[4] = c->headroom;
}
