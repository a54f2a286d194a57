// fp8q_device.h -- gfx950 device helpers: bf16 unpacking, E4M3 packing through the
// hardware converter, DPP lane reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8q_math.h"

#pragma clang fp contract(off)

namespace fp8q {

// ---------------------------------------------------------------- bf16 unpacking
// A 32-bit word holds two bf16 values: element 0 in bits 15:0, element 1 in 31:16.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ------------------------------------------------------------------ E4M3 packing
// gfx950's v_cvt_pk_fp8_f32 rounds binary32 to OCP E4M3 to nearest even; values are
// clipped to +-448 first so an out-of-range quotient saturates instead of becoming NaN.
__device__ __forceinline__ float clip448(float v) {
  return __builtin_amdgcn_fmed3f(v, -kE4M3Max, kE4M3Max);
}

// Four finite binary32 values -> four E4M3 codes, a in byte 0 ... d in byte 3.  With
// kSaturate the values are clipped to +-448 first; without it the caller guarantees
// |v| < 464: gfx950's v_cvt_pk_fp8_f32 rounds such magnitudes to at most 448 (464 is the
// midpoint between 448 and the NaN code's slot; farther out it produces the NaN code).
template <bool kSaturate>
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  if constexpr (kSaturate) {
    a = clip448(a); b = clip448(b); c = clip448(c); d = clip448(d);
  }
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return uint32_t(w);
}

// Eight bf16 (one 16-byte load) divided by a scale and packed into eight E4M3 codes.
//   kBounded: group quantization, every |x| <= amax and s = RN(max(amax, 1e-10) / 448).
//     Then |x / s| <= 448 / (1 - 2^-24), so RN(x / s) <= 448 + ulp(448): the estimate needs
//     no clip and the converter rounds the quotient to at most 448 (no saturation step).
//   otherwise: any scale (the KV cache's per-tensor scale may be far below |x| / 448): the
//     estimate is clipped so that inf - inf cannot occur and the result saturates at +-448.
template <bool kBounded>
__device__ __forceinline__ uint2 quant8(uint4 w, float s, float y) {
  auto dq = [&](float x) {
    return kBounded ? div_by_scale(x, s, y) : div_by_scale_clipped(x, s, y);
  };
  uint2 r;
  r.x = e4m3x4<!kBounded>(dq(bf16_lo(w.x)), dq(bf16_hi(w.x)), dq(bf16_lo(w.y)), dq(bf16_hi(w.y)));
  r.y = e4m3x4<!kBounded>(dq(bf16_lo(w.z)), dq(bf16_hi(w.z)), dq(bf16_lo(w.w)), dq(bf16_hi(w.w)));
  return r;
}

// ----------------------------------------------------------------- E4M3 decoding
// Two E4M3 codes (bytes 0,1 of w when kHigh is false, bytes 2,3 when true) -> binary32,
// exact (every E4M3 value, subnormals included, is a normal binary32).
template <bool kHigh>
__device__ __forceinline__ float2 e4m3x2_to_f32(uint32_t w) {
  const auto r = __builtin_amdgcn_cvt_pk_f32_fp8(int(w), kHigh);
  return make_float2(r[0], r[1]);
}

// binary32 -> bf16 bits, round to nearest even by integer carry (exact for every finite
// value whose rounding stays finite); any NaN becomes the quiet NaN 0x7FC0.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  return f != f ? 0x7FC0u : r;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Four E4M3 codes in w times a scale -> four bf16 packed in two 32-bit words (integer
// rounding; exact for NaN codes too).
__device__ __forceinline__ uint2 dequant4(uint32_t w, float s) {
  const float2 a = e4m3x2_to_f32<false>(w), b = e4m3x2_to_f32<true>(w);
  return make_uint2(pack_bf16x2(a.x * s, a.y * s), pack_bf16x2(b.x * s, b.y * s));
}

// Two binary32 -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32; used only on
// finite values (a NaN's bits are whatever the converter makes of it).
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// As dequant4, through the hardware converter: valid when no code of w is a NaN code.
__device__ __forceinline__ uint2 dequant4_finite(uint32_t w, float s) {
  const float2 a = e4m3x2_to_f32<false>(w), b = e4m3x2_to_f32<true>(w);
  return make_uint2(cvt_bf16x2(a.x * s, a.y * s), cvt_bf16x2(b.x * s, b.y * s));
}

// Non-zero iff one of the four codes in w is a NaN code (S.1111.111): adding 1 to the low
// seven bits of a byte carries into its top bit exactly when they are all ones.
__device__ __forceinline__ uint32_t e4m3_nan_bytes(uint32_t w) {
  return ((w & 0x7F7F7F7Fu) + 0x01010101u) & 0x80808080u;
}

// 16-byte load with the non-temporal (streaming) hint.
__device__ __forceinline__ uint4 load16_nt(const uint4* p) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// max |x| of eight bf16 packed in a 16-byte word, as binary32.
__device__ __forceinline__ float absmax8(uint4 w) {
  float m0 = fmaxf(fabsf(bf16_lo(w.x)), fabsf(bf16_hi(w.x)));
  float m1 = fmaxf(fabsf(bf16_lo(w.y)), fabsf(bf16_hi(w.y)));
  float m2 = fmaxf(fabsf(bf16_lo(w.z)), fabsf(bf16_hi(w.z)));
  float m3 = fmaxf(fabsf(bf16_lo(w.w)), fabsf(bf16_hi(w.w)));
  return fmaxf(fmaxf(m0, m1), fmaxf(m2, m3));
}

// --------------------------------------------------------------- DPP reductions
template <int kCtrl>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xF, 0xF,
                                                    false));
}

// Max over each aligned group of 8 lanes; every lane of the group gets the result.
__device__ __forceinline__ float max_over_8_lanes(float v) {
  v = fmaxf(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]: partner lane ^ 1
  v = fmaxf(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]: partner lane ^ 2
  v = fmaxf(v, dpp<0x141>(v));  // row_half_mirror: lane i <-> 7 - i within 8 lanes
  return v;
}

// Max over the whole 64-lane wave (result valid in every lane).
__device__ __forceinline__ float max_over_wave(float v) {
  v = max_over_8_lanes(v);
  v = fmaxf(v, dpp<0x140>(v));  // row_mirror: lane i <-> 15 - i within 16 lanes
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

}  // namespace fp8q
