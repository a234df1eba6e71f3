// OPQ quantize kernel (model card "OPQ INT4 Z-Image", sections "OPQ 原理" and
// "技术细节 / 存储格式"), per output row:
//   m = max_k |w|;  u = fl32(|w| / m);  q = round(15 u^alpha);  s = [w < 0];
//   packed nibbles eight per uint32, signs thirty-two per uint32.
//
// One wave owns one row.  The row is read from HBM once and held in VGPRs
// while the wave reduces the max, so HBM traffic is the algorithmic
// 2 B (bf16) read + 0.625 B written per weight.
//
// Exact codes without a device pow: the host gives the binary32 decision
// points T_k (code >= k  <=>  u >= T_k).  Positive binary32 values order like
// their bit patterns, so the code is a function of bits(u) that changes at
// fifteen points.  A table in LDS, indexed by the top bits of bits(u) (the
// host picks the coarsest grid that puts at most one decision point, with a
// guard band around it, in any bucket), gives for each bucket the number of
// decision points below it and the one that may fall inside it.
//
// Fast path: u' = |w| * fl32(1/m) instead of the division; u' is within 3 ulps
// of u, so comparing bits(u') with the bucket's point decides the code unless
// the two are within kGuard ulps.  Those rare elements (and every element of a
// row whose 1/m is not a normal number) redo the comparison with the correctly
// rounded quotient.
//
// A decision-point set that no grid separates (only for extreme alpha) falls
// back to counting against per-row magnitude thresholds: u >= T_k  <=>
// |w| >= A_k with A_k the smallest binary32 a such that fl32(a / m) >= T_k.
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

// ---------------------------------------------------------------- bucket table

constexpr uint32_t kGuard = 16;     // ulps around a decision point decided exactly
constexpr int kMaxBuckets = 2048;   // LDS words of the table
constexpr uint32_t kNoPoint = 0x7F000000u;  // above every bits(u'): never reached
constexpr int kMaxBlocks = 2048;    // grid of the table kernel (rows are strided)

// Bucket b covers bit patterns [b0 + (b << shift), b0 + ((b + 1) << shift)).
struct BucketGrid {
  uint32_t b0;
  int shift;
  int nb;
};

// The decision point's bit pattern with its low 4 bits replaced by 8: a table
// entry keeps bits 4..31 only; comparing against this centre and widening the
// guard by 8 covers every pattern that shares those bits.
__host__ __device__ inline uint32_t point_centre(float t) {
  uint32_t b;
  __builtin_memcpy(&b, &t, 4);
  return (b & ~15u) + 8u;
}
constexpr uint32_t kWindow = kGuard + 8;

// The coarsest grid (3..10 index bits per binade) on which the windows
// [centre - kWindow, centre + kWindow] of consecutive decision points never
// share a bucket.  False when none fits in kMaxBuckets.
bool bucket_grid(const DecisionPoints& dp, BucketGrid& g) {
  uint32_t c[kLevels];
  for (int j = 0; j < kLevels; ++j) c[j] = point_centre(dp.t[j]);
  if (c[0] <= 2 * kWindow) return false;
  const uint32_t top = 0x3F800000u + 64u;  // a little above bits(1.0f)
  for (int mbits = 3; mbits <= 10; ++mbits) {
    const int shift = 23 - mbits;
    const uint32_t b0 = (c[0] - kWindow) & ~((1u << shift) - 1u);
    if (b0 >= top) return false;
    const int64_t nb = (int64_t)((top - b0) >> shift) + 1;
    if (nb > kMaxBuckets) return false;
    bool ok = true;
    for (int j = 0; j + 1 < kLevels && ok; ++j)
      ok = ((c[j] + kWindow - b0) >> shift) < ((c[j + 1] - kWindow - b0) >> shift);
    if (ok) {
      g.b0 = b0;
      g.shift = shift;
      g.nb = (int)nb;
      return true;
    }
  }
  return false;
}

// Entry = (bits 4..31 of the point that may fall in the bucket, or kNoPoint)
// | (number of points wholly below the bucket).  Points are sorted, so the one
// that may fall inside is always number `below` (0-based).
__device__ void build_table(const DecisionPoints& dp, BucketGrid g, uint32_t* tab) {
  for (int b = threadIdx.x; b < g.nb; b += blockDim.x) {
    const uint32_t lo = g.b0 + ((uint32_t)b << g.shift);
    const uint32_t hi = lo + (1u << g.shift);
    uint32_t below = 0u;
#pragma unroll
    for (int j = 0; j < kLevels; ++j) below += (point_centre(dp.t[j]) + kWindow < lo) ? 1u : 0u;
    uint32_t e = kNoPoint | below;
    if (below < (uint32_t)kLevels) {
      const uint32_t c = point_centre(pick_point(dp, (int)below));
      if (c - kWindow < hi) e = (c - 8u) | below;
    }
    tab[b] = e;
  }
}

__device__ __forceinline__ uint32_t table_at(const uint32_t* tab, BucketGrid g, uint32_t ub) {
  const int b = (int)(ub - g.b0) >> g.shift;
  return tab[min(max(b, 0), g.nb - 1)];
}

// Exact code of magnitude a in a row with max m (any m >= a >= 0): the
// correctly rounded quotient, its bucket, and one comparison.
__device__ __forceinline__ uint32_t code_exact(float a, float m, const uint32_t* tab, BucketGrid g,
                                               const float* pts) {
  const float u = m > 0.0f ? a / m : 0.0f;
  const uint32_t e = table_at(tab, g, __float_as_uint(u));
  const uint32_t below = e & 15u;
  return below + ((below < (uint32_t)kLevels && u >= pts[below]) ? 1u : 0u);
}

template <typename T>
__device__ __forceinline__ uint32_t encode8_exact(const Slot<T>& s, float m, const uint32_t* tab,
                                                  BucketGrid g, const float* pts) {
  uint32_t word = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) word |= code_exact(fabsf(s.at(i)), m, tab, g, pts) << (4 * i);
  return word;
}

// Fast encode with u' = |x| * r; `amb` is set when some element lies within
// kWindow patterns of its bucket's point (the caller then re-encodes exactly).
template <typename T>
__device__ __forceinline__ uint32_t encode8_fast(const Slot<T>& s, float r, const uint32_t* tab,
                                                 BucketGrid g, bool& amb) {
  uint32_t word = 0u;
  bool near = false;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t ub = __float_as_uint(fabsf(s.at(i)) * r);
    const uint32_t e = table_at(tab, g, ub);
    const uint32_t c = (e & ~15u) | 8u;
    const uint32_t q = (e & 15u) + (ub >= c ? 1u : 0u);
    near |= (ub - c + kWindow) <= 2u * kWindow;
    word |= q << (4 * i);
  }
  amb = near;
  return word;
}

template <typename T>
__device__ __forceinline__ uint32_t sign_byte(const Slot<T>& s) {
  uint32_t sb = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) sb |= (s.at(i) < 0.0f ? 1u : 0u) << i;
  return sb;
}

template <typename T>
__device__ __forceinline__ uint32_t encode_chunk(const Slot<T>& v, float mx, float r, bool fast,
                                                 const uint32_t* tab, BucketGrid g,
                                                 const float* pts) {
  if (fast) {
    bool amb;
    const uint32_t word = encode8_fast(v, r, tab, g, amb);
    if (!amb) return word;
  }
  return encode8_exact(v, mx, tab, g, pts);
}

// Table kernel.  Blocks build the table once and stride over rows, one row per
// wave at a time.  NCH > 0: the row (k <= NCH * 512) stays in registers.
// NCH == 0: any k, the row is streamed twice (max pass, then encode pass).
template <typename T, int NCH>
__global__ __launch_bounds__(kRowsPerBlock * kWave) void quantize_rows_table(
    const T* __restrict__ w, int64_t n, int k, DecisionPoints dp, BucketGrid g,
    uint32_t* __restrict__ packed, uint32_t* __restrict__ sign, float* __restrict__ scale) {
  __shared__ uint32_t s_tab[kMaxBuckets];
  __shared__ float s_pts[kLevels + 1];
  build_table(dp, g, s_tab);
  if (threadIdx.x <= kLevels) s_pts[threadIdx.x] = threadIdx.x < kLevels ? pick_point(dp, threadIdx.x) : 2.0f;
  __syncthreads();

  const int lane = threadIdx.x & (kWave - 1);
  for (int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x / kWave); row < n;
       row += (int64_t)gridDim.x * kRowsPerBlock) {
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
      const bool fast = mx >= 0x1p-125f && mx <= 0x1p125f;  // 1/m normal, u' <= 1 + ulps
      const float r = 1.0f / mx;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int e0 = c * kChunk + lane * 8;
        const uint32_t word = encode_chunk(v[c], mx, r, fast, s_tab, g, s_pts);
        store_chunk(prow, srow, c, lane, e0 < k, word, sign_byte(v[c]));
      }
      if (lane == 0) scale[row] = mx;
    } else {
      const int nch = (k + kChunk - 1) / kChunk;
      float mx = 0.0f;
      for (int c = 0; c < nch; ++c) {
        const int e0 = c * kChunk + lane * 8;
        if (e0 < k) {
          Slot<T> sl;
          sl.load(wr + e0);
          mx = fmaxf(mx, slot_absmax(sl));
        }
      }
      mx = wave_max(mx);
      const bool fast = mx >= 0x1p-125f && mx <= 0x1p125f;
      const float r = 1.0f / mx;
      for (int c = 0; c < nch; ++c) {
        const int e0 = c * kChunk + lane * 8;
        Slot<T> sl;
        if (e0 < k) sl.load(wr + e0); else sl.zero();
        const uint32_t word = encode_chunk(sl, mx, r, fast, s_tab, g, s_pts);
        store_chunk(prow, srow, c, lane, e0 < k, word, sign_byte(sl));
      }
      if (lane == 0) scale[row] = mx;
    }
  }
}

// ---------------------------------------------------------------- threshold kernel (fallback)

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
  const int64_t groups = (n + kRowsPerBlock - 1) / kRowsPerBlock;
  BucketGrid g;
  if (bucket_grid(dp, g)) {
    const int64_t blocks = groups < kMaxBlocks ? groups : kMaxBlocks;
    hipLaunchKernelGGL((quantize_rows_table<T, NCH>), dim3((unsigned)blocks),
                       dim3(kRowsPerBlock * kWave), 0, stream, w, n, (int)k, dp, g, packed, sign,
                       scale);
  } else {
    hipLaunchKernelGGL((quantize_rows<T, NCH>), dim3((unsigned)groups),
                       dim3(kRowsPerBlock * kWave), 0, stream, w, n, (int)k, dp, packed, sign,
                       scale);
  }
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
