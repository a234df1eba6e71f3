// Device helpers shared by the libopq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "opq_internal.hpp"

namespace opq {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// binary32 -> bfloat16 bits, round to nearest even (finite inputs; values past
// the largest finite bfloat16 round to infinity as IEEE rounding does).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t b = __float_as_uint(f);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return b >> 16;
}

// double -> bfloat16 bits with a single rounding (nearest even).  The double is
// first rounded to binary32 with round-to-odd, which keeps enough bits (24 >= 8 + 2)
// for the second rounding to equal a direct one.
__device__ __forceinline__ uint32_t bf16_rne_from_f64(double d) {
  float f = (float)d;  // nearest even
  double back = (double)f;
  if (back != d) {
    uint32_t b = __float_as_uint(f);
    if (fabs(back) > fabs(d)) b -= 1u;  // step the magnitude back toward zero
    b |= 1u;                             // inexact: make the last bit odd
    f = __uint_as_float(b);
  }
  return bf16_rne(f);
}

// Reconstruction level selected by a lane-varying code without dynamic
// indexing into the by-value argument struct.
__device__ __forceinline__ double level_of(const Levels& lv, int q) {
  double g = 0.0;
#pragma unroll
  for (int i = 1; i <= kLevels; ++i) g = (q == i) ? lv.g[i] : g;
  return g;
}

// bfloat16 bits of the per-row table entry L[q] = bf16(G_q * m).
__device__ __forceinline__ uint32_t lut_entry(const Levels& lv, int q, float m) {
  return bf16_rne_from_f64(level_of(lv, q) * (double)m);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

}  // namespace opq
