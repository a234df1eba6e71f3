// OPQ quantize kernel (model card "OPQ INT4 Z-Image", sections "OPQ 原理" and
// "技术细节 / 存储格式"), per output row:
//   m = max_k |w|;  u = fl32(|w| / m);  q = round(15 u^alpha);  s = [w < 0];
//   packed nibbles eight per uint32, signs thirty-two per uint32.
//
// One wave owns one row.  The row is read from HBM once and held in VGPRs
// while the wave reduces the max, so HBM traffic is the algorithmic
// 2 B (bf16) read + 0.625 B written per weight.
//
// Exact codes without a device pow or a per-element division: the host gives
// the binary32 decision points T_k (code >= k  <=>  u >= T_k).  Because IEEE
// division rounds monotonically, u >= T_k  <=>  |w| >= A_k with
// A_k = the smallest binary32 a such that fl32(a / m) >= T_k.  Lanes 0..14 each
// find one A_k with a few correctly rounded divisions, then every element is
// compared against the fifteen row thresholds held in SGPRs.
#include "device_common.hpp"

namespace opq {
namespace {

constexpr int kRowsPerBlock = 4;       // one wave per row
constexpr int kChunk = kWave * 8;      // elements per wave-wide step (8 per lane)

// Eight consecutive elements of one lane, raw.
template <typename T>
struct Slot;
template <>
struct Slot<uint16_t> {
  uint32_t r[4];  // bf16 pairs, element 2i in the low half
  __device__ __forceinline__ void load(const uint16_t* p) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    r[0] = v.x; r[1] = v.y; r[2] = v.z; r[3] = v.w;
  }
  __device__ __forceinline__ void zero() { r[0] = r[1] = r[2] = r[3] = 0u; }
  __device__ __forceinline__ float at(int i) const {
    const uint32_t v = r[i >> 1];
    return __uint_as_float((i & 1) ? (v & 0xFFFF0000u) : (v << 16));
  }
};
template <>
struct Slot<float> {
  float r[8];
  __device__ __forceinline__ void load(const float* p) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
    r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = 0.0f;
  }
  __device__ __forceinline__ float at(int i) const { return r[i]; }
};

template <typename T>
__device__ __forceinline__ float slot_absmax(const Slot<T>& s) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(s.at(i)));
  return m;
}

__device__ __forceinline__ float next_up(float a) { return __uint_as_float(__float_as_uint(a) + 1u); }
__device__ __forceinline__ float next_down(float a) { return __uint_as_float(__float_as_uint(a) - 1u); }

// Smallest binary32 a >= 0 with fl32(a / m) >= t, for finite m > 0, t in (0, 1].
// fl32(t * m) is within a couple of ulps of it; the loops walk the rest with
// correctly rounded divisions.
__device__ float magnitude_threshold(float t, float m) {
  float a = t * m;
  for (int it = 0; it < 32 && !(a / m >= t); ++it) a = next_up(a);
  for (int it = 0; it < 32 && a > 0.0f && (next_down(a) / m >= t); ++it) a = next_down(a);
  return a;
}

__device__ __forceinline__ float pick_point(const DecisionPoints& dp, int j) {
  float t = dp.t[0];
#pragma unroll
  for (int i = 1; i < kLevels; ++i) t = (j == i) ? dp.t[i] : t;
  return t;
}

// Encode one lane's eight elements: returns the packed word, sets the sign byte.
template <typename T>
__device__ __forceinline__ uint32_t encode8(const Slot<T>& s, const float (&A)[kLevels],
                                            uint32_t& signs) {
  uint32_t word = 0u, sb = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float x = s.at(i);
    const float ax = fabsf(x);
    uint32_t q = 0u;
#pragma unroll
    for (int j = 0; j < kLevels; ++j) q += (ax >= A[j]) ? 1u : 0u;
    word |= q << (4 * i);
    sb |= (x < 0.0f ? 1u : 0u) << i;
  }
  signs = sb;
  return word;
}

// Row thresholds A_1..A_15, uniform across the wave.
__device__ __forceinline__ void row_thresholds(const DecisionPoints& dp, float m, int lane,
                                               float (&A)[kLevels]) {
  float a = __builtin_inff();
  if (m > 0.0f && lane < kLevels) a = magnitude_threshold(pick_point(dp, lane), m);
#pragma unroll
  for (int j = 0; j < kLevels; ++j) A[j] = readlane_f(a, j);
}

// Store one chunk's packed word and the sign word shared by four lanes.
__device__ __forceinline__ void store_chunk(uint32_t* prow, uint32_t* srow, int c, int lane,
                                            bool valid, uint32_t word, uint32_t sbyte) {
  uint32_t s32 = valid ? (sbyte << (8 * (lane & 3))) : 0u;
  s32 |= __shfl_xor(s32, 1, kWave);
  s32 |= __shfl_xor(s32, 2, kWave);
  if (valid) {
    prow[c * kWave + lane] = word;
    if ((lane & 3) == 0) srow[c * (kChunk / 32) + (lane >> 2)] = s32;
  }
}

// NCH > 0: the row (k <= NCH * 512) stays in registers.  NCH == 0: any k, the
// row is streamed twice (max pass, then encode pass).
template <typename T, int NCH>
__global__ __launch_bounds__(kRowsPerBlock * kWave) void quantize_rows(
    const T* __restrict__ w, int64_t n, int k, DecisionPoints dp, uint32_t* __restrict__ packed,
    uint32_t* __restrict__ sign, float* __restrict__ scale) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x / kWave);
  if (row >= n) return;  // whole waves leave; no block-wide barrier below
  const T* wr = w + row * (int64_t)k;
  uint32_t* prow = packed + row * (int64_t)(k / 8);
  uint32_t* srow = sign + row * (int64_t)(k / 32);

  if constexpr (NCH > 0) {
    Slot<T> v[NCH];
    float mx = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int e0 = c * kChunk + lane * 8;
      if (e0 < k) {
        v[c].load(wr + e0);
        mx = fmaxf(mx, slot_absmax(v[c]));
      } else {
        v[c].zero();
      }
    }
    mx = wave_max(mx);
    float A[kLevels];
    row_thresholds(dp, mx, lane, A);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int e0 = c * kChunk + lane * 8;
      uint32_t sb;
      const uint32_t word = encode8(v[c], A, sb);
      store_chunk(prow, srow, c, lane, e0 < k, word, sb);
    }
    if (lane == 0) scale[row] = mx;
  } else {
    const int nch = (k + kChunk - 1) / kChunk;
    float mx = 0.0f;
    for (int c = 0; c < nch; ++c) {
      const int e0 = c * kChunk + lane * 8;
      if (e0 < k) {
        Slot<T> s;
        s.load(wr + e0);
        mx = fmaxf(mx, slot_absmax(s));
      }
    }
    mx = wave_max(mx);
    float A[kLevels];
    row_thresholds(dp, mx, lane, A);
    for (int c = 0; c < nch; ++c) {
      const int e0 = c * kChunk + lane * 8;
      Slot<T> s;
      if (e0 < k) s.load(wr + e0); else s.zero();
      uint32_t sb;
      const uint32_t word = encode8(s, A, sb);
      store_chunk(prow, srow, c, lane, e0 < k, word, sb);
    }
    if (lane == 0) scale[row] = mx;
  }
}

template <typename T, int NCH>
hipError_t launch_rows(const T* w, int64_t n, int64_t k, const DecisionPoints& dp,
                       uint32_t* packed, uint32_t* sign, float* scale, hipStream_t stream) {
  const int64_t blocks = (n + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL((quantize_rows<T, NCH>), dim3((unsigned)blocks), dim3(kRowsPerBlock * kWave),
                     0, stream, w, n, (int)k, dp, packed, sign, scale);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch(const T* w, int64_t n, int64_t k, const DecisionPoints& dp, uint32_t* packed,
                    uint32_t* sign, float* scale, hipStream_t stream) {
  const int64_t nch = (k + kChunk - 1) / kChunk;
  // bf16 slots take 4 VGPRs per chunk, fp32 slots 8: fp32 rows stay in
  // registers up to 16 chunks, bf16 rows up to 32.
  if (nch <= 1) return launch_rows<T, 1>(w, n, k, dp, packed, sign, scale, stream);
  if (nch <= 2) return launch_rows<T, 2>(w, n, k, dp, packed, sign, scale, stream);
  if (nch <= 4) return launch_rows<T, 4>(w, n, k, dp, packed, sign, scale, stream);
  if (nch <= 8) return launch_rows<T, 8>(w, n, k, dp, packed, sign, scale, stream);
  if (nch <= 12) return launch_rows<T, 12>(w, n, k, dp, packed, sign, scale, stream);
  if (nch <= 16) return launch_rows<T, 16>(w, n, k, dp, packed, sign, scale, stream);
  if constexpr (sizeof(T) == 2) {
    if (nch <= 20) return launch_rows<T, 20>(w, n, k, dp, packed, sign, scale, stream);
    if (nch <= 24) return launch_rows<T, 24>(w, n, k, dp, packed, sign, scale, stream);
    if (nch <= 32) return launch_rows<T, 32>(w, n, k, dp, packed, sign, scale, stream);
  }
  return launch_rows<T, 0>(w, n, k, dp, packed, sign, scale, stream);
}

}  // namespace

hipError_t launch_quantize(const void* w, bool w_is_bf16, int64_t n, int64_t k,
                           const DecisionPoints& dp, uint32_t* packed, uint32_t* sign,
                           float* scale, hipStream_t stream) {
  if (w_is_bf16)
    return dispatch(static_cast<const uint16_t*>(w), n, k, dp, packed, sign, scale, stream);
  return dispatch(static_cast<const float*>(w), n, k, dp, packed, sign, scale, stream);
}

}  // namespace opq
