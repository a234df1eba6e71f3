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

// One-touch streams.  The kernels read each weight and write each code, sign
// and reconstructed value exactly once; such accesses carry the nontemporal
// hint (`nt`), so the streams do not displace reusable lines in the L2 and the
// Infinity Cache.  Measured on this part with inputs rotated past the 256 MB
// Infinity Cache: dequantize 8 % faster on large layers (20 % on a 3840 x 3840
// weight) with its stores marked, quantize 1-10 % with its loads and stores
// marked.  Loads are marked only where the data is read once.
__device__ __forceinline__ void store_stream(uint32_t* p, uint32_t v) {
  __builtin_nontemporal_store(v, p);
}
__device__ __forceinline__ void store_stream16(void* p, uint32_t a, uint32_t b, uint32_t c,
                                               uint32_t d) {
  const u32x4_t v = {a, b, c, d};
  __builtin_nontemporal_store(v, static_cast<u32x4_t*>(p));
}
__device__ __forceinline__ u32x4_t load_stream16(const void* p) {
  return __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
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

// Block barrier for data exchanged through LDS only.  The release fence makes
// the wave's LDS writes complete (lgkmcnt 0) and, with the acquire fence after
// the barrier, keeps the compiler from moving any LDS access across it; global
// loads in flight stay in flight, which a full __syncthreads would wait for.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The same barrier for kernels that also fill LDS with direct-to-LDS loads
// (global_load_lds).  The release fence above would wait for every such load
// still in flight (they write LDS too); here the caller waits (vmcnt) for the
// loads whose data the barrier publishes, this wave's own LDS accesses complete
// (lgkmcnt 0), and empty asm statements that clobber memory keep the compiler
// from moving any memory access across the barrier.
__device__ __forceinline__ void lds_barrier_dma() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS written by some lanes of a wave and read by others of the same wave: the
// wave's LDS operations are done in issue order, so the wait and the
// wavefront-scope fence (which orders the accesses for the compiler) suffice.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront", "local");
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
