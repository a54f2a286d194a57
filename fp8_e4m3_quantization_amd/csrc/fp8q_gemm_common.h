// fp8q_gemm_common.h -- pieces shared by the persistent decode GEMM kernels (W8A8 and
// W8A16): MFMA operand vector types, the projection set one launch walks, the strip
// lookup, buffer descriptors for the weight stream and the LDS-only barrier.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kMaxProj = 8;  // projections of one activation in one launch
constexpr int kPWaves = 8;   // waves of a persistent workgroup (one workgroup per CU)

// Several projections that read the same activation: output strips of 16 columns are
// numbered across them in order.
struct ProjSet {
  const uint8_t* w[kMaxProj];
  const float* ws[kMaxProj];
  uint16_t* out[kMaxProj];
  int ldc[kMaxProj];
  int strip_end[kMaxProj];  // cumulative strip count after projection p
  int count;
};

// strip s -> (projection, first column); uniform across the workgroup
__device__ __forceinline__ void locate_strip(const ProjSet& ps, int s, int* p_out, int* n0) {
  int p = 0;
  while (p + 1 < ps.count && s >= ps.strip_end[p]) ++p;
  *p_out = p;
  *n0 = (s - (p ? ps.strip_end[p - 1] : 0)) * 16;
}

// s_waitcnt lgkmcnt(0) + s_barrier: orders the LDS partials without waiting on the
// weight prefetches that are still in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt untouched
  __builtin_amdgcn_s_barrier();
}

// Weight loads go through a buffer descriptor per strip (base = the strip's first row,
// 16*k bytes).  A strip past the end gets a zero-size descriptor: its loads return zeros
// without touching memory, so every prefetch is issued unconditionally and the compiler
// tracks the in-order load counter exactly (no branch around any load).
constexpr uint32_t kBufferDword3 = 0x00020000;  // raw 32-bit buffer format (gfx9 family)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_strip_rsrc(const uint8_t* base, int k,
                                                                  bool valid) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, valid ? 16 * k : 0,
                                           kBufferDword3);
}

// Weight block scales are read-only for the whole launch and uniform per wave: reading
// them through the constant address space makes them scalar loads (counted apart from
// the vector weight loads, so waiting for a scale never drains the weight prefetch).
typedef const __attribute__((address_space(4))) float const_float;

// 32 bytes at byte offset off of a buffer, as eight dwords (two 16-byte loads).
template <int kAux>
__device__ __forceinline__ v8i buffer_load32(__amdgpu_buffer_rsrc_t r, int off) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kAux);
  const v4u y = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, kAux);
  v8i o;
  o[0] = int(x[0]); o[1] = int(x[1]); o[2] = int(x[2]); o[3] = int(x[3]);
  o[4] = int(y[0]); o[5] = int(y[1]); o[6] = int(y[2]); o[7] = int(y[3]);
  return o;
}

}  // namespace fp8q
