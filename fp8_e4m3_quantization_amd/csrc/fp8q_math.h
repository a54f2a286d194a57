// fp8q_math.h -- scalar arithmetic shared by the HIP kernels (device) and by the host
// side of the library (and its CPU proof harness).  Plain C++: builds under hipcc for
// gfx950 and under a host C++ compiler.
//
// Division by a scale.  Every quantizer on the path divides a bf16 value by an fp32 scale
// in IEEE binary32 (one correctly rounded division) before rounding to E4M3
// (fp8_act_quant.rs page, module doc: all variants must emit identical bytes;
// fp8_calibration.rs page, module doc: scale = amax * headroom / 448).  A full
// correctly-rounded division costs ~10 VALU instructions on gfx950, so per element the
// kernels instead use the reciprocal y = RN(1/s) (computed once per scale) and one
// remainder correction:
//     q  = RN(x * y)
//     r' = RN(q * s - x)        (fma; the negated remainder)
//     q1 = RN(q - r' * y)       (fma)
// q1 equals RN(x / s) for every bf16 x and every binary32 s >= 2^-64, as long as the
// quotient is at least 2^-11 and no larger than 1024; below 2^-11 both round to a
// signed E4M3 zero; above 1024 both saturate.  The identity holds because all three
// steps are exact scalings of one another across binades, so it is a statement about the
// 2^7 bf16 mantissas times the 2^23 binary32 mantissas of s, which the test suite
// checks exhaustively on the CPU.  Writing the remainder with its sign flipped keeps a
// negative zero input negative (a -0 sum would otherwise round to +0).
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define FP8Q_HD __host__ __device__
#else
#define FP8Q_HD
#endif

namespace fp8q {

// IEEE binary32 max finite OCP E4M3 value.
constexpr float kE4M3Max = 448.0f;
// Floor applied to an all-zero (or tiny) amax before dividing by 448.
constexpr float kAmaxFloor = 1e-10f;

FP8Q_HD inline float bits_to_f32(uint32_t b) {
  union { uint32_t u; float f; } c;
  c.u = b;
  return c.f;
}

FP8Q_HD inline uint32_t f32_to_bits(float f) {
  union { uint32_t u; float f; } c;
  c.f = f;
  return c.u;
}

// x / s rounded to nearest-even, given y = RN(1/s); see the header comment for its range.
FP8Q_HD inline float div_by_scale(float x, float s, float y) {
  float q = x * y;
  float rn = __builtin_fmaf(q, s, -x);
  return __builtin_fmaf(-rn, y, q);
}

// As above, but first clips the estimate to +-1024 so that a quotient far beyond the
// E4M3 range can never produce inf - inf; the result then still lies beyond +-448.
FP8Q_HD inline float div_by_scale_clipped(float x, float s, float y) {
  float q = x * y;
#if defined(__HIP_DEVICE_COMPILE__)
  q = __builtin_amdgcn_fmed3f(q, -1024.0f, 1024.0f);  // one v_med3_f32; same for non-NaN q
#else
  q = q > 1024.0f ? 1024.0f : (q < -1024.0f ? -1024.0f : q);
#endif
  float rn = __builtin_fmaf(q, s, -x);
  return __builtin_fmaf(-rn, y, q);
}

// bf16 (bit pattern) widened to fp32, exact.
FP8Q_HD inline float bf16_to_f32(uint16_t h) { return bits_to_f32(uint32_t(h) << 16); }

// fp32 -> bf16 bit pattern, round to nearest even (finite inputs).
FP8Q_HD inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t b = f32_to_bits(f);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return uint16_t(b >> 16);
}

// Per-group scale: max(amax, 1e-10) / 448, correctly rounded.  amax is a bf16 magnitude
// (or the floor), so the division uses the same remainder-corrected product with the
// constant RN(1/448).  The floor is not a bf16 value, so its quotient is a constant.
FP8Q_HD inline float group_scale_from_amax(float amax) {
  constexpr float kInv448 = 1.0f / 448.0f;                 // RN(1/448), folded exactly
  constexpr float kFloorScale = kAmaxFloor / kE4M3Max;     // RN(1e-10f / 448)
  float s = div_by_scale(amax, kE4M3Max, kInv448);
  return amax > kAmaxFloor ? s : kFloorScale;
}

}  // namespace fp8q
