// Exhaustive CPU check of the library's per-element division (fp8q_math.h): for every
// bf16 mantissa of x and every binary32 mantissa of s, the remainder-corrected product
// must equal the correctly rounded quotient x / s.  All three operations scale exactly
// across binades while they stay normal, so one binade of x and s covers every exponent
// pair in the range the kernels use; a randomized pass over exponents backs that up.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>

#include "fp8q_math.h"

using fp8q::bits_to_f32;
using fp8q::f32_to_bits;

int main() {
  long long bad = 0;
  // 1) one binade: x in [1,2) with 7 stored bits, s in [1,2) with 23 stored bits
#pragma omp parallel for reduction(+ : bad) schedule(static)
  for (int sm = 0; sm < (1 << 23); ++sm) {
    float s = bits_to_f32(0x3F800000u | uint32_t(sm));
    float y = 1.0f / s;
    for (int xm = 0; xm < 128; ++xm) {
      float x = bits_to_f32(0x3F800000u | (uint32_t(xm) << 16));
      float want = x / s;
      float got = fp8q::div_by_scale(x, s, y);
      float gotc = fp8q::div_by_scale_clipped(x, s, y);
      float gotn = fp8q::div_by_scale(-x, s, y);
      if (f32_to_bits(got) != f32_to_bits(want) || f32_to_bits(gotc) != f32_to_bits(want) ||
          f32_to_bits(gotn) != f32_to_bits(-want))
        ++bad;
    }
  }
  printf("binade_mismatches %lld\n", bad);
  long long bad2 = 0;
  // 2) random exponents: quotient in [2^-11, 2^10], s >= 2^-64
  std::mt19937_64 rng(12345);
  for (int i = 0; i < 20000000; ++i) {
    uint32_t xb = uint32_t(rng() & 0x7FFF) << 16;
    if ((xb >> 23) == 0xFF || (xb >> 23) == 0) continue;
    float x = bits_to_f32(xb);
    int qexp = int(rng() % 22) - 11;  // target quotient exponent
    int sexp = int((xb >> 23)) - 127 - qexp;
    if (sexp < -64 || sexp > 127) continue;
    uint32_t sb = (uint32_t(sexp + 127) << 23) | uint32_t(rng() & 0x7FFFFF);
    float s = bits_to_f32(sb);
    float y = 1.0f / s;
    if (f32_to_bits(fp8q::div_by_scale(x, s, y)) != f32_to_bits(x / s)) ++bad2;
  }
  printf("random_exponent_mismatches %lld\n", bad2);
  // 3) signed zeros keep their sign
  long long bad3 = 0;
  for (int sm = 0; sm < 1000; ++sm) {
    float s = bits_to_f32(0x3F800000u | uint32_t(sm * 7919));
    float y = 1.0f / s;
    if (f32_to_bits(fp8q::div_by_scale(-0.0f, s, y)) != 0x80000000u) ++bad3;
    if (f32_to_bits(fp8q::div_by_scale(0.0f, s, y)) != 0u) ++bad3;
  }
  printf("signed_zero_mismatches %lld\n", bad3);
  // 4) the group scale: every positive finite bf16 amax (and zero) against max(a,1e-10)/448
  long long bad4 = 0;
  for (uint32_t h = 0; h < 0x7F80; ++h) {
    float a = fp8q::bf16_to_f32(uint16_t(h));
    float want = (a > 1e-10f ? a : 1e-10f) / 448.0f;
    if (f32_to_bits(fp8q::group_scale_from_amax(a)) != f32_to_bits(want)) ++bad4;
  }
  printf("group_scale_mismatches %lld\n", bad4);
  // 5) clipped form: quotients far beyond the range saturate with the right sign
  long long bad5 = 0;
  for (int i = 0; i < 1000000; ++i) {
    float x = bits_to_f32((uint32_t(rng() % 0x7F7F) + 1) << 16);
    float s = bits_to_f32(uint32_t(rng() % 0x7F7FFFFF) + 0x00800000u);
    if (!(std::isfinite(x) && std::isfinite(s)) || s <= 0) continue;
    float y = 1.0f / s;
    if (!std::isfinite(y) || y == 0) continue;
    double exact = double(x) / double(s);
    if (exact <= 1024.0) continue;
    float g = fp8q::div_by_scale_clipped(x, s, y);
    float gn = fp8q::div_by_scale_clipped(-x, s, y);
    if (!(g >= 464.0f) || !(gn <= -464.0f)) ++bad5;
  }
  printf("saturation_mismatches %lld\n", bad5);
  return (bad || bad2 || bad3 || bad4 || bad5) ? 1 : 0;
}
