// Group-wise scales: the stored form of the model card "OPQ INT4 Z-Image"
// ("技术细节 / 存储格式": one float16 max per group of weights, the
// configuration section offering groups of 32, 64, 128 or 256; "推理解码": the
// decode multiplies by that group max).  A group is `gs` consecutive weights
// of a row along k; its stored max m16 is max|w| rounded to float16 (nearest,
// ties to even, saturated at 65504); codes are taken against m16 and a code q
// stands for bf16(G_q m16).
#pragma once

#include "decode.hpp"

namespace opq {

constexpr int kMantissas = 1024;  // float16 significands

// float16 bits of x (0 <= x, finite), rounded to nearest even and saturated
// at 65504.  Written out in integer arithmetic, so the result does not depend
// on the hardware's float16 denormal mode.
__device__ __forceinline__ uint32_t f16_bits_rn(float x) {
  x = fminf(x, 65504.0f);
  if (x >= 0x1p-14f) {
    const uint32_t b = __float_as_uint(x);
    return ((b + 0xFFFu + ((b >> 13) & 1u)) >> 13) - (112u << 10);
  }
  // subnormal float16: j 2^-24 with j = rint(x 2^24); j = 1024 is 2^-14's bits
  return (uint32_t)__builtin_rintf(x * 0x1p24f);
}

// The float16 value with bits h (finite, sign clear), exactly, as binary32.
__device__ __forceinline__ float f16_value(uint32_t h) {
  const uint32_t e = (h >> 10) & 31u, mt = h & 1023u;
  return e ? __uint_as_float(((e + 112u) << 23) | (mt << 13)) : (float)mt * 0x1p-24f;
}

// T[mt][q] = bf16(G_q (1 + mt/1024)), q = 0..15, as eight words of bf16 pairs
// (entries 2j, 2j+1 in word j) per significand: one row per float16
// significand.  A group's table is the row of its stored max with the max's
// exponent added, since scaling by a power of two commutes with rounding while
// the results stay normal (the host checks G_1 2^-24 >= 2^-126).
__device__ __forceinline__ void build_mant_table(const Levels& lv, uint32_t* tab) {
  for (int mt = threadIdx.x; mt < kMantissas; mt += blockDim.x) {
    const double mm = 1.0 + (double)mt * (1.0 / kMantissas);
    uint32_t d[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      d[j] = bf16_rne_from_f64(lv.g[2 * j] * mm) | (bf16_rne_from_f64(lv.g[2 * j + 1] * mm) << 16);
    *reinterpret_cast<u32x4_t*>(tab + 8 * mt) = u32x4_t{d[0], d[1], d[2], d[3]};
    *reinterpret_cast<u32x4_t*>(tab + 8 * mt + 4) = u32x4_t{d[4], d[5], d[6], d[7]};
  }
}

typedef unsigned short g16x2_t __attribute__((ext_vector_type(2)));

// Byte planes of the table of a group with stored max bits h.
__device__ __forceinline__ RowLut group_lut(const uint32_t* tab, uint32_t h) {
  const uint32_t fb = __float_as_uint(f16_value(h));
  const uint32_t mt = (fb >> 13) & 1023u;
  const uint32_t e16 = ((fb >> 16) - (127u << 7)) & 0xFF80u;  // (exponent - 127) << 7, mod 2^16
  const uint32_t add = e16 | (e16 << 16);
  const u32x4_t a = *reinterpret_cast<const u32x4_t*>(tab + 8 * mt);
  const u32x4_t b = *reinterpret_cast<const u32x4_t*>(tab + 8 * mt + 4);
  uint32_t d[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  const uint32_t live = fb ? 0xFFFFFFFFu : 0u;  // a zero max gives an all-zero table
#pragma unroll
  for (int j = 0; j < 8; ++j)
    d[j] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(g16x2_t, d[j]) +
                                            __builtin_bit_cast(g16x2_t, add)) & live;
  d[0] &= 0xFFFF0000u;  // L[0] = +0
  RowLut t;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    t.lo[i] = __builtin_amdgcn_perm(d[2 * i + 1], d[2 * i], 0x06040200u);
    t.hi[i] = __builtin_amdgcn_perm(d[2 * i + 1], d[2 * i], 0x07050301u);
  }
  return t;
}

}  // namespace opq
