// OPQ quantize kernel (model card "OPQ INT4 Z-Image", sections "OPQ 原理" and
// "技术细节 / 存储格式"), per output row:
//   m = max_k |w|;  u = fl32(|w| / m);  q = round(15 u^alpha);  s = [w < 0];
//   packed nibbles eight per uint32, signs thirty-two per uint32.
//
// A block of 256 threads owns one row at a time (one wave per row in the
// kernels for rows of up to 2048 or more than 16384 elements).  The row is read from HBM once and held
// in VGPRs while the max is reduced, so HBM traffic is the algorithmic 2 B
// (bf16) read + 0.625 B written per weight.  Both streams are one-touch and go
// nontemporal (load_once, store_stream), except in the kernels that read a long
// row twice, whose second pass should find the row in cache.
//
// The file also holds the variants of the same encoder: the error sums of the
// alpha sweep (codes reconstructed and compared instead of stored), the
// group-wise form (a float16 max per group of weights) and 3/5/6-bit codes.
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
#include "group.hpp"

#include <algorithm>
#include <atomic>

namespace opq {
namespace {

constexpr int kRowsPerBlock = 4;       // one wave per row
constexpr int kChunk = kWave * 8;      // elements per wave-wide step (8 per lane)

typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, a),
                                                                 __builtin_bit_cast(u16x2_t, b)));
}

// Eight consecutive elements of one lane, raw.
template <typename T>
struct Slot;
template <>
struct Slot<uint16_t> {
  typedef uint32_t Acc;  // running max of |w|: two bf16 magnitude patterns
  uint32_t r[4];         // bf16 pairs, element 2i in the low half
  __device__ __forceinline__ void load(const uint16_t* p) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    r[0] = v.x; r[1] = v.y; r[2] = v.z; r[3] = v.w;
  }
  // The same for data read only once (nontemporal).
  __device__ __forceinline__ void load_once(const uint16_t* p) {
    const u32x4_t v = load_stream16(p);
    r[0] = v.x; r[1] = v.y; r[2] = v.z; r[3] = v.w;
  }
  __device__ __forceinline__ void zero() { r[0] = r[1] = r[2] = r[3] = 0u; }
  // Element i widened to binary32 (exact).
  __device__ __forceinline__ float at(int i) const {
    const uint32_t v = r[i >> 1];
    return __uint_as_float((i & 1) ? (v & 0xFFFF0000u) : (v << 16));
  }
  // w_i < 0 on the raw pattern: sign set and magnitude not zero (-0.0 is not < 0).
  __device__ __forceinline__ bool neg(int i) const {
    const uint32_t v = r[i >> 1];
    return (i & 1) ? (v > 0x8000FFFFu) : ((uint16_t)v > (uint16_t)0x8000u);
  }
  __device__ __forceinline__ static Acc acc0() { return 0u; }
  __device__ __forceinline__ void absmax(Acc& a) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) a = pk_max_u16(a, r[j] & 0x7FFF7FFFu);
  }
  __device__ __forceinline__ static float finish(Acc a) {
    return __uint_as_float(max(a & 0xFFFFu, a >> 16) << 16);
  }
};
template <>
struct Slot<float> {
  typedef float Acc;
  float r[8];
  __device__ __forceinline__ void load(const float* p) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
    r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
  }
  __device__ __forceinline__ void load_once(const float* p) {
    const u32x4_t a = load_stream16(p), b = load_stream16(p + 4);
    r[0] = __uint_as_float(a.x); r[1] = __uint_as_float(a.y);
    r[2] = __uint_as_float(a.z); r[3] = __uint_as_float(a.w);
    r[4] = __uint_as_float(b.x); r[5] = __uint_as_float(b.y);
    r[6] = __uint_as_float(b.z); r[7] = __uint_as_float(b.w);
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = 0.0f;
  }
  __device__ __forceinline__ float at(int i) const { return r[i]; }
  __device__ __forceinline__ bool neg(int i) const { return r[i] < 0.0f; }
  __device__ __forceinline__ static Acc acc0() { return 0.0f; }
  __device__ __forceinline__ void absmax(Acc& a) const {
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(r[i]));
  }
  __device__ __forceinline__ static float finish(Acc a) { return a; }
};

template <typename T>
__device__ __forceinline__ float slot_absmax(const Slot<T>& s) {
  typename Slot<T>::Acc a = Slot<T>::acc0();
  s.absmax(a);
  return Slot<T>::finish(a);
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

// Sign bits of one lane's eight elements (bit i = [w_i < 0]).
template <typename T>
__device__ __forceinline__ uint32_t sign_byte(const Slot<T>& s) {
  uint32_t sb = 0u;
#pragma unroll
  for (int i = 7; i >= 0; --i) sb = (sb << 1) + (s.neg(i) ? 1u : 0u);
  return sb;
}
// bfloat16 pairs, four instructions a pair instead of six: adding 0x7FFF to a
// half's magnitude sets its top bit exactly when the magnitude is not zero
// (no carry crosses into the other half), so r & that & 0x80008000 keeps the
// sign bits of the halves with w < 0 (-0.0 gives 0); v_dot4_u32_u8 then sums
// those bytes (0x80 or 0) with weights 2^i at element i's byte.
template <>
__device__ __forceinline__ uint32_t sign_byte(const Slot<uint16_t>& s) {
  constexpr uint32_t kWeights[4] = {0x02000100u, 0x08000400u, 0x20001000u, 0x80004000u};
  uint32_t acc = 0u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t r = s.r[j];
    const uint32_t nz = (r & 0x7FFF7FFFu) + 0x7FFF7FFFu;
    acc = __builtin_amdgcn_udot4(r & nz & 0x80008000u, kWeights[j], acc, false);
  }
  return acc >> 7;
}

// Store one chunk's packed word and the sign word shared by four lanes.
__device__ __forceinline__ void store_chunk(uint32_t* prow, uint32_t* srow, int c, int lane,
                                            bool valid, uint32_t word, uint32_t sbyte) {
  uint32_t s32 = valid ? (sbyte << (8 * (lane & 3))) : 0u;
  // OR over each group of four lanes (quad permutes 1,0,3,2 and 2,3,0,1)
  s32 |= (uint32_t)__builtin_amdgcn_mov_dpp((int)s32, 0xB1, 0xF, 0xF, false);
  s32 |= (uint32_t)__builtin_amdgcn_mov_dpp((int)s32, 0x4E, 0xF, 0xF, false);
  if (valid) {
    store_stream(prow + c * kWave + lane, word);
    if ((lane & 3) == 0) store_stream(srow + c * (kChunk / 32) + (lane >> 2), s32);
  }
}

// ---------------------------------------------------------------- bucket table

constexpr uint32_t kGuard = 16;             // ulps around a decision point decided exactly
constexpr int kMaxBuckets = 1024;           // 8-byte entries
constexpr uint32_t kNoPoint = 0x7F000000u;  // above every clamped bits(u')
constexpr uint32_t kTop = 0x40000000u;      // bits(2.0f): u' is clamped to [floor, 2]
constexpr int kMaxBlocks = 2048;            // grid of the error-sum table kernel (rows are strided)
// Grid of the code table kernel: a row to a wave up to 32768 rows, strided
// beyond.  Measured against a cap of 2048 blocks (8192 waves, some taking two
// rows and some one) on bf16 rows of 3840, same box, interleaved: 11520 rows
// 26.3 -> 25.8 us, 20480 rows 41.3 -> 39.5 us.
constexpr int kMaxRowBlocks = 8192;

// Buckets b = 0 .. nb-1 cover bit patterns [b0 + (b << shift), b0 + ((b + 1) << shift));
// the last one reaches past bits(2.0f).  b0 is a multiple of 2^shift, and the
// table has `size` slots (nb rounded up to a power of two) with bucket b in
// slot ((b0 >> shift) + b) mod size, so a bit pattern's slot is
// (bits >> shift) mod size: its byte offset (bits >> (shift - 3)) & mask8 is
// two instructions, with no base to subtract.
struct BucketGrid {
  uint32_t b0;
  int shift;
  int nb;
  int size;
};

inline int table_slots(int64_t nb) {
  int s = 1;
  while (s < nb) s *= 2;
  return s;
}

__host__ __device__ inline uint32_t float_bits(float t) {
  uint32_t b;
  __builtin_memcpy(&b, &t, 4);
  return b;
}

// The coarsest grid (3..10 index bits per binade) on which the windows
// [bits(T_j) - kGuard, bits(T_j) + kGuard] of consecutive decision points never
// share a bucket.  False when none fits in kMaxBuckets.
bool bucket_grid(const DecisionPoints& dp, BucketGrid& g) {
  uint32_t c[kLevels];
  for (int j = 0; j < kLevels; ++j) c[j] = float_bits(dp.t[j]);
  if (c[0] <= 2 * kGuard) return false;
  for (int mbits = 3; mbits <= 10; ++mbits) {
    const int shift = 23 - mbits;
    const uint32_t b0 = (c[0] - kGuard) & ~((1u << shift) - 1u);
    const int64_t nb = (int64_t)((kTop - b0) >> shift) + 1;
    if (nb > kMaxBuckets) return false;
    bool ok = true;
    for (int j = 0; j + 1 < kLevels && ok; ++j)
      ok = ((c[j] + kGuard - b0) >> shift) < ((c[j + 1] - kGuard - b0) >> shift);
    if (ok) {
      g.b0 = b0;
      g.shift = shift;
      g.nb = (int)nb;
      g.size = table_slots(nb);
      return true;
    }
  }
  return false;
}

// Entry b: y = number of decision points wholly below the bucket (their guard
// windows end before it); x = kGuard - bits(T_y) when point y's window reaches
// into the bucket, kGuard - kNoPoint otherwise (arithmetic mod 2^32).  Points
// are sorted, so only point y can reach in.  For a clamped u' in the bucket,
// d = bits(u') + x = bits(u') - bits(T_y) + kGuard fits an int32:
//   code = y + [d >= kGuard],  decided exactly unless 0 <= d <= 2 kGuard.
// The fast encoder takes [d >= kGuard] from the carry of the 32-bit sum
// bits(u') + x, which is set exactly when bits(u') >= bits(T_y) - kGuard (x is
// 2^32 - (bits(T_y) - kGuard), and bits(T_y) > 2 kGuard; never for kNoPoint):
// the two agree everywhere outside [bits(T_y) - kGuard, bits(T_y) + kGuard],
// and inside it d <= 2 kGuard sends the element to the exact re-encode.  One
// add with carry-out then replaces an add and a compare.
__device__ void build_table(const DecisionPoints& dp, BucketGrid g, uint2* tab) {
  for (int b = threadIdx.x; b < g.nb; b += blockDim.x) {
    const uint32_t lo = g.b0 + ((uint32_t)b << g.shift);
    const uint32_t hi = lo + (1u << g.shift);
    // Static indices only: a lane-dependent index into dp would become a
    // load from the argument segment.
    uint32_t below = 0u, next = kNoPoint;
#pragma unroll
    for (int j = kLevels - 1; j >= 0; --j) {
      const uint32_t c = float_bits(dp.t[j]);
      const bool under = c + kGuard < lo;
      below += under ? 1u : 0u;
      next = under ? next : c;  // ends at the lowest point not wholly below
    }
    const uint32_t x = (next != kNoPoint && next - kGuard < hi) ? kGuard - next : kGuard - kNoPoint;
    tab[((g.b0 >> g.shift) + (uint32_t)b) & (uint32_t)(g.size - 1)] = make_uint2(x, below);
  }
}

// Table entry for a quotient already clamped to [floor, 2.0]; sh3 is the
// grid's shift - 3 and mask8 is (size - 1) * 8.
__device__ __forceinline__ uint2 table_at(const uint2* tab, uint32_t ub, int sh3, uint32_t mask8) {
  const uint32_t off = (ub >> sh3) & mask8;
  return *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(tab) + off);
}

// Exact code of magnitude a in a row with max m (m >= a >= 0): the correctly
// rounded quotient, its bucket, and one comparison with the next point
// (pts[15] = 2 is never reached).
__device__ __forceinline__ uint32_t code_exact(float a, float m, const uint2* tab, int sh3,
                                               uint32_t mask8, float ulo, const float* pts) {
  const float u = m > 0.0f ? a / m : 0.0f;
  const float uc = fminf(fmaxf(u, ulo), 2.0f);
  const uint32_t below = table_at(tab, __float_as_uint(uc), sh3, mask8).y;
  return below + (u >= pts[below] ? 1u : 0u);
}

template <typename T>
__device__ __forceinline__ uint32_t encode8_exact(const Slot<T>& s, float m, const uint2* tab,
                                                  int sh3, uint32_t mask8, float ulo,
                                                  const float* pts) {
  uint32_t word = 0u;
#pragma unroll
  for (int i = 7; i >= 0; --i) {
    // an opaque copy keeps |w| from being formed ahead of the branch (the fast
    // path folds it into its multiply)
    float v = s.at(i);
    asm volatile("" : "+v"(v));
    word = (word << 4) + code_exact(fabsf(v), m, tab, sh3, mask8, ulo, pts);
  }
  return word;
}

// Fast encode with u' = |w| * r (r = fl32(1/m), u' within 3 ulps of u), clamped
// to [floor, 2].  `near` ends at min over the elements of the unsigned d; the
// caller re-encodes exactly when it is <= 2 kGuard.
template <typename T>
__device__ __forceinline__ uint32_t encode8_fast(const Slot<T>& s, float r, const uint2* tab,
                                                 int sh3, uint32_t mask8, float ulo,
                                                 uint32_t& near) {
  uint32_t word = 0u, nr = 0xFFFFFFFFu;
#pragma unroll
  for (int i = 7; i >= 0; --i) {
    // finite here: the row max is normal and 1/m too
    const float up = __builtin_amdgcn_fmed3f(fabsf(s.at(i)) * r, ulo, 2.0f);
    const uint32_t ub = __float_as_uint(up);
    const uint2 e = table_at(tab, ub, sh3, mask8);
    uint32_t d;
    const uint32_t up_step = __builtin_add_overflow(ub, e.x, &d) ? 1u : 0u;
    word = (word << 4) + e.y + up_step;
    nr = min(nr, d);
  }
  near = nr;
  return word;
}

template <typename T>
__device__ __forceinline__ uint32_t encode_chunk(const Slot<T>& v, float mx, float r, bool fast,
                                                 const uint2* tab, int sh3, uint32_t mask8,
                                                 float ulo, const float* pts) {
  // The fast encode runs on every chunk (with 1 standing in for 1/m where it
  // does not apply), so the exact re-encode is the only branch.
  uint32_t near;
  uint32_t word = encode8_fast(v, fast ? r : 1.0f, tab, sh3, mask8, ulo, near);
  if (!fast || near <= 2u * kGuard) word = encode8_exact(v, mx, tab, sh3, mask8, ulo, pts);
  return word;
}

// Codes of a lane's eight elements (fast path, then exact where flagged).
template <typename T>
__device__ __forceinline__ void codes8(const Slot<T>& v, float mx, float r, bool fast,
                                       const uint2* tab, int sh3, uint32_t mask8, float ulo,
                                       const float* pts, uint32_t (&q)[8]) {
  // As encode_chunk: the fast path runs everywhere, the exact one where flagged.
  const float rf = fast ? r : 1.0f;
  uint32_t nr = fast ? 0xFFFFFFFFu : 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float up = __builtin_amdgcn_fmed3f(fabsf(v.at(i)) * rf, ulo, 2.0f);
    const uint32_t ub = __float_as_uint(up);
    const uint2 e = table_at(tab, ub, sh3, mask8);
    uint32_t d;
    const uint32_t up_step = __builtin_add_overflow(ub, e.x, &d) ? 1u : 0u;  // as in encode8_fast
    q[i] = e.y + up_step;
    nr = min(nr, d);
  }
  if (nr <= 2u * kGuard) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float x = v.at(i);
      asm volatile("" : "+v"(x));
      q[i] = code_exact(fabsf(x), mx, tab, sh3, mask8, ulo, pts);
    }
  }
}

// Table kernel: blocks build the table, then each wave takes one row at a time
// (rows strided over the grid).  NCH > 0: the row (k <= NCH * 512) stays in
// registers; this is the kernel for rows of up to 2048 elements, and for
// bfloat16 rows of up to 4096 when there are many rows (see dispatch).
// NCH == 0: any k, the row is streamed twice (max, then encode); it takes rows
// longer than the block kernel's 16384.
template <typename T, int NCH>
__global__ __launch_bounds__(kRowsPerBlock * kWave) void quantize_rows_table(
    const T* __restrict__ w, int64_t n, int k, DecisionPoints dp, BucketGrid g,
    uint32_t* __restrict__ packed, uint32_t* __restrict__ sign, float* __restrict__ scale) {
  __shared__ uint2 s_tab[kMaxBuckets];
  __shared__ float s_pts[kLevels + 1];
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t stride = (int64_t)gridDim.x * kRowsPerBlock;
  int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x / kWave);

  // The first row's loads go out before the table is built.
  Slot<T> v[NCH > 0 ? NCH : 1];
  auto load_row = [&](int64_t rr) {
    const T* wr = w + rr * (int64_t)k;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int e0 = c * kChunk + lane * 8;
      if (e0 < k) v[c].load_once(wr + e0); else v[c].zero();
    }
  };
  if constexpr (NCH > 0) {
    if (row < n) load_row(row);
  }

  build_table(dp, g, s_tab);
  if (threadIdx.x == 0) {
#pragma unroll
    for (int j = 0; j < kLevels; ++j) s_pts[j] = dp.t[j];
    s_pts[kLevels] = 2.0f;
  }
  // The table is in LDS once lgkmcnt drains; the row loads stay in flight
  // (a full __syncthreads would wait for them too).
  lds_barrier();
  const int sh3 = g.shift - 3;
  const uint32_t mask8 = (uint32_t)(g.size - 1) << 3;
  const float ulo = __uint_as_float(g.b0);

  for (; row < n; row += stride) {
    uint32_t* prow = packed + row * (int64_t)(k / 8);
    uint32_t* srow = sign + row * (int64_t)(k / 32);
    if constexpr (NCH > 0) {
      typename Slot<T>::Acc acc = Slot<T>::acc0();
#pragma unroll
      for (int c = 0; c < NCH; ++c) v[c].absmax(acc);
      const float mx = wave_max(Slot<T>::finish(acc));
      const bool fast = mx >= 0x1p-125f && mx <= 0x1p125f;  // 1/m normal, u' <= 1 + ulps
      const float r = 1.0f / mx;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int e0 = c * kChunk + lane * 8;
        const uint32_t word = encode_chunk(v[c], mx, r, fast, s_tab, sh3, mask8, ulo, s_pts);
        store_chunk(prow, srow, c, lane, e0 < k, word, sign_byte(v[c]));
      }
      if (lane == 0) scale[row] = mx;
      if (row + stride < n) load_row(row + stride);
    } else {
      const T* wr = w + row * (int64_t)k;
      const int nch = (k + kChunk - 1) / kChunk;
      typename Slot<T>::Acc acc = Slot<T>::acc0();
      for (int c = 0; c < nch; ++c) {
        const int e0 = c * kChunk + lane * 8;
        if (e0 < k) {
          Slot<T> sl;
          sl.load(wr + e0);
          sl.absmax(acc);
        }
      }
      const float mx = wave_max(Slot<T>::finish(acc));
      const bool fast = mx >= 0x1p-125f && mx <= 0x1p125f;
      const float r = 1.0f / mx;
      for (int c = 0; c < nch; ++c) {
        const int e0 = c * kChunk + lane * 8;
        Slot<T> sl;
        if (e0 < k) sl.load(wr + e0); else sl.zero();
        const uint32_t word = encode_chunk(sl, mx, r, fast, s_tab, sh3, mask8, ulo, s_pts);
        store_chunk(prow, srow, c, lane, e0 < k, word, sign_byte(sl));
      }
      if (lane == 0) scale[row] = mx;
    }
  }
}

// Error sums over rows of up to 2048 elements, one wave per row (the row in
// registers, rows strided over the grid), for the same reason as the table
// kernel above: the codes as there, each element then reconstructed from the
// row's table L[q] = bf16(G_q m) in the wave's own LDS slot (a wave's LDS
// operations complete in order, so no block barrier), and the row's
// (sum w^2, sum (w - w')^2) accumulated in binary32 per lane and across the
// wave (at most 2048 nonnegative terms), written as doubles.  Elements past k
// are zero and add nothing.
template <typename T, int NCH>
__global__ __launch_bounds__(kRowsPerBlock * kWave) void error_rows_table(
    const T* __restrict__ w, int64_t n, int k, DecisionPoints dp, BucketGrid g, Levels lv,
    double* __restrict__ row_sums) {
  __shared__ uint2 s_tab[kMaxBuckets];
  __shared__ float s_pts[kLevels + 1];
  __shared__ uint32_t s_recw[kRowsPerBlock][16];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int64_t stride = (int64_t)gridDim.x * kRowsPerBlock;
  int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + wave;

  Slot<T> v[NCH];
  auto load_row = [&](int64_t rr) {
    const T* wr = w + rr * (int64_t)k;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int e0 = c * kChunk + lane * 8;
      if (e0 < k) v[c].load_once(wr + e0); else v[c].zero();
    }
  };
  if (row < n) load_row(row);

  build_table(dp, g, s_tab);
  if (threadIdx.x == 0) {
#pragma unroll
    for (int j = 0; j < kLevels; ++j) s_pts[j] = dp.t[j];
    s_pts[kLevels] = 2.0f;
  }
  lds_barrier();
  const int sh3 = g.shift - 3;
  const uint32_t mask8 = (uint32_t)(g.size - 1) << 3;
  const float ulo = __uint_as_float(g.b0);

  for (; row < n; row += stride) {
    typename Slot<T>::Acc acc = Slot<T>::acc0();
#pragma unroll
    for (int c = 0; c < NCH; ++c) v[c].absmax(acc);
    const float mx = wave_max(Slot<T>::finish(acc));
    const bool fast = mx >= 0x1p-125f && mx <= 0x1p125f;  // 1/m normal, u' <= 1 + ulps
    const float r = 1.0f / mx;
    if (lane < 16) s_recw[wave][lane] = lut_entry(lv, lane, mx);
    wave_lds_sync();
    float sw2 = 0.0f, se2 = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      // the codes themselves (no packed word to take apart again)
      uint32_t q[8];
      codes8(v[c], mx, r, fast, s_tab, sh3, mask8, ulo, s_pts, q);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float xv = v[c].at(i);
        // a nonzero code carries the weight's sign, so |w - w'| = ||w| - L[q]|
        const float e = fabsf(xv) - __uint_as_float(s_recw[wave][q[i]] << 16);
        sw2 = fmaf(xv, xv, sw2);
        se2 = fmaf(e, e, se2);
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      sw2 += __shfl_xor(sw2, off, kWave);
      se2 += __shfl_xor(se2, off, kWave);
    }
    if (lane == 0) {
      row_sums[2 * row] = (double)sw2;
      row_sums[2 * row + 1] = (double)se2;
    }
    if (row + stride < n) load_row(row + stride);
  }
}

// ---------------------------------------------------------------- block-per-row kernel
//
// A block of 256 threads owns one row at a time: thread t holds elements
// c*2048 + 8t .. c*2048 + 8t + 7 of chunk c (NCT chunks, k <= NCT * 2048), so a
// wave's share of a row is a quarter of the one-wave-per-row kernel's and the
// encode tail after the last load is short.  Blocks stride over rows (the
// grid is twice the resident count); the next row's loads are issued before
// the current row is encoded, into the other register buffer.  When that grid
// covers every row, each block takes one row and keeps no second buffer.  The
// row max meets in LDS behind a barrier that waits for LDS traffic only, so
// those loads stay in flight.

constexpr int kBlockThreads = 256;
constexpr int kBlockChunk = kBlockThreads * 8;  // elements per block-wide chunk

// Store word `wi` of a row and, from the first lane of each quad, the sign word
// wi / 4 made of the quad's four sign bytes.
__device__ __forceinline__ void store_word(uint32_t* prow, uint32_t* srow, int wi, int lane,
                                           bool valid, uint32_t word, uint32_t sbyte) {
  uint32_t s32 = valid ? (sbyte << (8 * (lane & 3))) : 0u;
  s32 |= (uint32_t)__builtin_amdgcn_mov_dpp((int)s32, 0xB1, 0xF, 0xF, false);
  s32 |= (uint32_t)__builtin_amdgcn_mov_dpp((int)s32, 0x4E, 0xF, 0xF, false);
  if (valid) {
    store_stream(prow + wi, word);
    if ((lane & 3) == 0) store_stream(srow + (wi >> 2), s32);
  }
}

// kErr: instead of storing the stored form, reconstruct every element as
// opq_dequantize would (the row's table L[q] = bf16(G_q m) built in LDS once the
// max is known) and write the row's (sum w^2, sum (w - w')^2): binary32 per lane
// over its at most 64 elements and across the wave, then double across the
// block's waves in a fixed order.
// kOne: the grid has a block per row, so there is no next row to prefetch and
// one register buffer (8 fewer VGPRs for bfloat16 rows of two chunks, which
// lets 8 instead of 7 blocks share a CU).
template <typename T, int NCT, bool kErr, bool kOne = false>
__global__ __launch_bounds__(kBlockThreads) void quantize_block_rows(
    const T* __restrict__ w, int64_t n, int k, DecisionPoints dp, BucketGrid g,
    uint32_t* __restrict__ packed, uint32_t* __restrict__ sign, float* __restrict__ scale,
    Levels lv, double* __restrict__ row_sums) {
  __shared__ uint2 s_tab[kMaxBuckets];
  __shared__ float s_pts[kLevels + 1];
  __shared__ float s_wmax[2][kBlockThreads / kWave];
  __shared__ double s_sum[2][kBlockThreads / kWave][2];
  __shared__ uint32_t s_recw[kBlockThreads / kWave][16];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int64_t stride = gridDim.x;

  Slot<T> v[kOne ? 1 : 2][NCT];
  auto load_row = [&](int64_t rr, int buf) __attribute__((always_inline)) {
    const T* wr = w + rr * (int64_t)k;
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      const int e0 = c * kBlockChunk + tid * 8;
      if (e0 < k) v[buf][c].load_once(wr + e0); else v[buf][c].zero();
    }
  };
  int64_t row = blockIdx.x;
  if (row < n) load_row(row, 0);

  // No barrier here: the first row-max barrier below comes before any read
  // of the table or the points.
  build_table(dp, g, s_tab);
  if (tid == 0) {
#pragma unroll
    for (int j = 0; j < kLevels; ++j) s_pts[j] = dp.t[j];
    s_pts[kLevels] = 2.0f;
  }
  const int sh3 = g.shift - 3;
  const uint32_t mask8 = (uint32_t)(g.size - 1) << 3;
  const float ulo = __uint_as_float(g.b0);

  // Encode the row held in buffer `buf`; `ms` picks the LDS slot of its max
  // (slots alternate, so one barrier per row keeps writes after old reads).
  int64_t pend = -1;  // row whose partial sums wait in s_sum (kErr)
  auto flush_sums = [&](int slot) __attribute__((always_inline)) {
    if (tid == 0 && pend >= 0) {
      double a0 = 0.0, a1 = 0.0;
#pragma unroll
      for (int q = 0; q < kBlockThreads / kWave; ++q) {
        a0 += s_sum[slot][q][0];
        a1 += s_sum[slot][q][1];
      }
      row_sums[2 * pend] = a0;
      row_sums[2 * pend + 1] = a1;
    }
  };
  auto process = [&](int64_t rr, int buf, int ms) __attribute__((always_inline)) {
    typename Slot<T>::Acc acc = Slot<T>::acc0();
#pragma unroll
    for (int c = 0; c < NCT; ++c) v[buf][c].absmax(acc);
    float mx = wave_max(Slot<T>::finish(acc));
    if (lane == 0) s_wmax[ms][wave] = mx;
    lds_barrier();
    mx = s_wmax[ms][0];
#pragma unroll
    for (int q = 1; q < kBlockThreads / kWave; ++q) mx = fmaxf(mx, s_wmax[ms][q]);
    if constexpr (kErr) flush_sums(ms ^ 1);
    const bool fast = mx >= 0x1p-125f && mx <= 0x1p125f;  // 1/m normal, u' <= 1 + ulps
    const float r = 1.0f / mx;
    if constexpr (!kErr) {
      uint32_t* prow = packed + rr * (int64_t)(k / 8);
      uint32_t* srow = sign + rr * (int64_t)(k / 32);
#pragma unroll
      for (int c = 0; c < NCT; ++c) {
        const int e0 = c * kBlockChunk + tid * 8;
        const uint32_t word = encode_chunk(v[buf][c], mx, r, fast, s_tab, sh3, mask8, ulo, s_pts);
        store_word(prow, srow, e0 >> 3, lane, e0 < k, word, sign_byte(v[buf][c]));
      }
      if (tid == 0) scale[rr] = mx;
    } else {
      // Each wave writes the row's table L[q] = bf16(G_q m) into its own LDS
      // slot (lanes 0..15 one entry each): LDS ops of one wave complete in
      // order, so no block barrier is needed before the lookups.
      if (lane < 16) s_recw[wave][lane] = lut_entry(lv, lane, mx);
      wave_lds_sync();
      float sw2 = 0.0f, se2 = 0.0f;
#pragma unroll
      for (int c = 0; c < NCT; ++c) {
        // the codes themselves (no packed word to take apart again)
        uint32_t q[8];
        codes8(v[buf][c], mx, r, fast, s_tab, sh3, mask8, ulo, s_pts, q);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float xv = v[buf][c].at(i);  // zero past k
          // a nonzero code carries the weight's sign, so |w - w'| = ||w| - L[q]|
          const float e = fabsf(xv) - __uint_as_float(s_recw[wave][q[i]] << 16);
          sw2 = fmaf(xv, xv, sw2);
          se2 = fmaf(e, e, se2);
        }
      }
      // binary32 over the wave (at most 64 x 64 positive terms: relative
      // error below 70 * 2^-24), double across the block's waves
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        sw2 += __shfl_xor(sw2, off, kWave);
        se2 += __shfl_xor(se2, off, kWave);
      }
      const double d0 = sw2, d1 = se2;
      // The block's partials are summed after the next row's barrier (or the
      // one after the loop); slots alternate with the rows.
      if (lane == 0) {
        s_sum[ms][wave][0] = d0;
        s_sum[ms][wave][1] = d1;
      }
      pend = rr;
    }
  };

  if constexpr (kOne) {
    if (row < n) process(row, 0, 0);
  } else if constexpr (kErr) {
    // One copy of the row code, the prefetched row moved into buffer 0 after
    // each row: 70 instead of 86 VGPRs for bfloat16 rows of two chunks, and
    // 8-10 % faster (for the codes themselves it measured slower).
    int ms = 0;
    while (row < n) {
      const int64_t r1 = row + stride;
      if (r1 < n) load_row(r1, 1);
      process(row, 0, ms);
#pragma unroll
      for (int c = 0; c < NCT; ++c) v[0][c] = v[1][c];
      ms ^= 1;
      row = r1;
    }
  } else {
    // Rows alternate between the two buffers (register arrays need constant indices).
    while (row < n) {
      const int64_t r1 = row + stride;
      if (r1 < n) load_row(r1, 1);
      process(row, 0, 0);
      if (r1 >= n) break;
      const int64_t r2 = r1 + stride;
      if (r2 < n) load_row(r2, 0);
      process(r1, 1, 1);
      row = r2;
    }
  }
  if constexpr (kErr) {
    // the last row's partials: which slot holds them follows the row count
    lds_barrier();
    const int64_t cnt = blockIdx.x < n ? (n - 1 - blockIdx.x) / stride + 1 : 0;
    flush_sums((int)((cnt - 1) & 1));
  }
}

// Encode against per-row magnitude thresholds A_1..A_15 (fallback kernel).
template <typename T>
__device__ __forceinline__ uint32_t encode8(const Slot<T>& s, const float (&A)[kLevels]) {
  uint32_t word = 0u;
#pragma unroll
  for (int i = 7; i >= 0; --i) {
    const float ax = fabsf(s.at(i));
    uint32_t q = 0u;
#pragma unroll
    for (int j = 0; j < kLevels; ++j) q += (ax >= A[j]) ? 1u : 0u;
    word = (word << 4) + q;
  }
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
        v[c].load_once(wr + e0);
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
      store_chunk(prow, srow, c, lane, e0 < k, encode8(v[c], A), sign_byte(v[c]));
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
      store_chunk(prow, srow, c, lane, e0 < k, encode8(s, A), sign_byte(s));
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
    const int64_t blocks = groups < kMaxRowBlocks ? groups : kMaxRowBlocks;
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

// Blocks of the strided kernel that fit on the device at once (the grid must
// not exceed it: a block waiting for a slot would start only after another
// block had finished all of its rows).  Per-CU occupancy is computed once per
// kernel; the CU count is asked of the current device per call.
template <typename T, int NCT, bool kErr, bool kOne = false>
int64_t resident_blocks() {
  static const int per_cu = [] {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, quantize_block_rows<T, NCT, kErr, kOne>,
                                                     kBlockThreads, 0) != hipSuccess || b < 1)
      b = 1;
    return b;
  }();
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 1;
  return (int64_t)per_cu * cus;
}

template <typename T, int NCT, bool kErr = false>
hipError_t launch_block_rows(const T* w, int64_t n, int64_t k, const DecisionPoints& dp,
                             const BucketGrid& g, uint32_t* packed, uint32_t* sign, float* scale,
                             hipStream_t stream, const Levels* lv = nullptr,
                             double* row_sums = nullptr) {
  // Twice the blocks that fit at once: the second half starts as the first
  // finishes, which evens out the rows per block (15.8 -> 14.4 us for a
  // 3840 x 3840 bf16 weight, no loss at 11520 rows).  When that many blocks
  // cover every row, a block per row without the prefetch buffer; for the
  // codes up to four times the resident count (7680 x 3840 bf16: 24.7 ->
  // 23.0 us; equal at 11520 rows, 2% slower at 20480).
  Levels lvv{};
  if (lv) lvv = *lv;
  if (n <= (kErr ? 2 : 4) * resident_blocks<T, NCT, kErr, true>()) {
    hipLaunchKernelGGL((quantize_block_rows<T, NCT, kErr, true>), dim3((unsigned)n),
                       dim3(kBlockThreads), 0, stream, w, n, (int)k, dp, g, packed, sign, scale,
                       lvv, row_sums);
    return hipGetLastError();
  }
  const int64_t blocks = 2 * resident_blocks<T, NCT, kErr>();
  hipLaunchKernelGGL((quantize_block_rows<T, NCT, kErr>), dim3((unsigned)blocks),
                     dim3(kBlockThreads), 0, stream, w, n, (int)k, dp, g, packed, sign, scale,
                     lvv, row_sums);
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch_error(const T* w, int64_t n, int64_t k, const DecisionPoints& dp,
                          const Levels& lv, double* row_sums, hipStream_t stream) {
  BucketGrid g;
  if (!bucket_grid(dp, g)) return hipErrorNotSupported;
  // rows of up to 2048 elements one to a wave, as for the codes
  const int64_t nch = (k + kChunk - 1) / kChunk;
  if (nch <= 4) {
    const int64_t groups = (n + kRowsPerBlock - 1) / kRowsPerBlock;
    const dim3 grid((unsigned)(groups < kMaxBlocks ? groups : kMaxBlocks));
    const dim3 block(kRowsPerBlock * kWave);
    if (nch <= 1)
      hipLaunchKernelGGL((error_rows_table<T, 1>), grid, block, 0, stream, w, n, (int)k, dp, g, lv, row_sums);
    else if (nch <= 2)
      hipLaunchKernelGGL((error_rows_table<T, 2>), grid, block, 0, stream, w, n, (int)k, dp, g, lv, row_sums);
    else
      hipLaunchKernelGGL((error_rows_table<T, 4>), grid, block, 0, stream, w, n, (int)k, dp, g, lv, row_sums);
    return hipGetLastError();
  }
  const int64_t nct = (k + kBlockChunk - 1) / kBlockChunk;
#define OPQ_ERR_CASE(N)                                                                        \
  if (nct <= N)                                                                                \
    return launch_block_rows<T, N, true>(w, n, k, dp, g, nullptr, nullptr, nullptr, stream, &lv, \
                                         row_sums);
  OPQ_ERR_CASE(2) OPQ_ERR_CASE(3) OPQ_ERR_CASE(4) OPQ_ERR_CASE(5)
  OPQ_ERR_CASE(6) OPQ_ERR_CASE(8)
#undef OPQ_ERR_CASE
  return hipErrorNotSupported;
}

constexpr int64_t kWaveRowsMin = 8192;

template <typename T>
hipError_t dispatch(const T* w, int64_t n, int64_t k, const DecisionPoints& dp, uint32_t* packed,
                    uint32_t* sign, float* scale, hipStream_t stream) {
  const int64_t nch = (k + kChunk - 1) / kChunk;
  BucketGrid g;
  // Rows of up to 2048 elements go one to a wave (below, through the table
  // kernel): a 256-thread block would leave threads idle on them (11520 x 1024
  // bf16: 18.2 -> 10.7 us).  bfloat16 rows of up to 4096 elements go one to a
  // wave as well when there are at least kWaveRowsMin of them (at least two
  // rows per resident wave of that kernel, 112 VGPRs): no block barrier or LDS
  // exchange per row (11520 x 3840 29.1-29.3 -> 27.3-28.9 us, 20480 x 3840
  // 49.1-50.6 -> 49.1-49.2); with fewer rows the block per row is faster
  // (3840 x 3840 11.7-12.1 against 12.5 us), four times the lanes on each row
  // shortening the tail.
  const bool wave_rows = sizeof(T) == 2 && nch <= 8 && n >= kWaveRowsMin;
  if (nch > 4 && !wave_rows && bucket_grid(dp, g)) {
    const int64_t nct = (k + kBlockChunk - 1) / kBlockChunk;
    if (nct <= 2) return launch_block_rows<T, 2>(w, n, k, dp, g, packed, sign, scale, stream);
    if (nct <= 3) return launch_block_rows<T, 3>(w, n, k, dp, g, packed, sign, scale, stream);
    if (nct <= 4) return launch_block_rows<T, 4>(w, n, k, dp, g, packed, sign, scale, stream);
    if (nct <= 5) return launch_block_rows<T, 5>(w, n, k, dp, g, packed, sign, scale, stream);
    if (nct <= 6) return launch_block_rows<T, 6>(w, n, k, dp, g, packed, sign, scale, stream);
    if (nct <= 8) return launch_block_rows<T, 8>(w, n, k, dp, g, packed, sign, scale, stream);
  }
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

// ---------------------------------------------------------------- group-wise form
//
// The weights stream as one flat array of n*k elements.  A wave takes 512
// consecutive elements (8 per lane) at a time; groups never straddle them
// (gs divides both 512 and k), so a group is gs/8 consecutive lanes and its
// max comes from a butterfly over those lanes.  The codes are then found as in
// the row kernels, against the stored float16 max, whose reciprocal is exact
// enough for the fast path because m16 >= 2^-24 is a normal binary32.  After
// the table build there is no block barrier: waves run independently.
constexpr int kGThreads = 256;
constexpr int kGWaves = kGThreads / kWave;
constexpr int kGUnroll = 2;  // chunks per wave per batch

template <typename T, int GS>
__global__ __launch_bounds__(kGThreads) void quantize_grouped_rows(
    const T* __restrict__ w, int64_t total, DecisionPoints dp, BucketGrid g,
    uint32_t* __restrict__ packed, uint32_t* __restrict__ sign, uint16_t* __restrict__ scale16) {
  static_assert(GS >= 32 && GS <= 256 && (GS & (GS - 1)) == 0, "group of 32..256");
  constexpr int kLanes = GS / 8;  // lanes per group
  __shared__ uint2 s_tab[kMaxBuckets];
  __shared__ float s_pts[kLevels + 1];
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t nchunks = (total + kChunk - 1) / kChunk;
  const int64_t wid = (int64_t)blockIdx.x * kGWaves + threadIdx.x / kWave;

  // The grid has one batch of kGUnroll chunks per wave.
  Slot<T> v[kGUnroll];
  const int64_t cb = wid * kGUnroll;  // first chunk of this wave's batch
  if (cb < nchunks) {
#pragma unroll
    for (int u = 0; u < kGUnroll; ++u) {
      const int64_t e0 = (cb + u) * kChunk + lane * 8;
      if (e0 < total) v[u].load_once(w + e0); else v[u].zero();
    }
  }

  build_table(dp, g, s_tab);
  if (threadIdx.x == 0) {
#pragma unroll
    for (int j = 0; j < kLevels; ++j) s_pts[j] = dp.t[j];
    s_pts[kLevels] = 2.0f;
  }
  lds_barrier();
  const int sh3 = g.shift - 3;
  const uint32_t mask8 = (uint32_t)(g.size - 1) << 3;
  const float ulo = __uint_as_float(g.b0);

  if (cb >= nchunks) return;  // after the barrier: the block's table is shared
#pragma unroll
  for (int u = 0; u < kGUnroll; ++u) {
    const int64_t e0 = (cb + u) * kChunk + lane * 8;
    const bool valid = e0 < total;
    float mx = slot_absmax(v[u]);
#pragma unroll
    for (int off = 1; off < kLanes; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, kWave));
    const uint32_t h = f16_bits_rn(mx);
    const float m16 = f16_value(h);
    const bool fast = m16 > 0.0f;
    const float r = fast ? 1.0f / m16 : 0.0f;
    const uint32_t word = encode_chunk(v[u], m16, r, fast, s_tab, sh3, mask8, ulo, s_pts);
    const int64_t wi = valid ? (e0 >> 3) : 0;
    store_word(packed + wi, sign + (wi >> 2), 0, lane, valid, word, sign_byte(v[u]));
    if (valid && lane % kLanes == 0) scale16[e0 / GS] = (uint16_t)h;
  }
}

template <typename T, int GS>
hipError_t launch_grouped_rows(const T* w, int64_t n, int64_t k, const DecisionPoints& dp,
                               const BucketGrid& g, uint32_t* packed, uint32_t* sign,
                               uint16_t* scale16, hipStream_t stream) {
  // One batch per wave: with the grid capped at the resident block count (and
  // the waves looping), a 11520 x 3840 weight took 35.9 us instead of 32.2.
  // Inputs past the 32-bit grid go in several launches of whole rows (groups
  // never straddle rows).
  const int64_t per_batch = (int64_t)kChunk * kGUnroll;
  const int64_t max_rows = std::max<int64_t>(1, kMaxLaunchThreads / kWave * per_batch / k);
  for (int64_t r0 = 0; r0 < n; r0 += max_rows) {
    const int64_t total = std::min(max_rows, n - r0) * k;
    const int64_t batches = (total + per_batch - 1) / per_batch;
    const int64_t blocks = (batches + kGWaves - 1) / kGWaves;
    hipLaunchKernelGGL((quantize_grouped_rows<T, GS>), dim3((unsigned)blocks), dim3(kGThreads), 0,
                       stream, w + r0 * k, total, dp, g, packed + r0 * (k / 8),
                       sign + r0 * (k / 32), scale16 + r0 * (k / GS));
  }
  return hipGetLastError();
}

template <typename T>
hipError_t dispatch_grouped(const T* w, int64_t n, int64_t k, int gs, const DecisionPoints& dp,
                            uint32_t* packed, uint32_t* sign, uint16_t* scale16,
                            hipStream_t stream) {
  BucketGrid g;
  if (!bucket_grid(dp, g)) return hipErrorNotSupported;
  switch (gs) {
    case 32: return launch_grouped_rows<T, 32>(w, n, k, dp, g, packed, sign, scale16, stream);
    case 64: return launch_grouped_rows<T, 64>(w, n, k, dp, g, packed, sign, scale16, stream);
    case 128: return launch_grouped_rows<T, 128>(w, n, k, dp, g, packed, sign, scale16, stream);
    case 256: return launch_grouped_rows<T, 256>(w, n, k, dp, g, packed, sign, scale16, stream);
    default: return hipErrorInvalidValue;
  }
}

// ---------------------------------------------------------------- other code widths
//
// b-bit codes (the configuration section's 3, 5 or 6 bits; 2^b - 1 levels in
// place of 15).  Same structure as quantize_block_rows: a block owns a row at
// a time, the row stays in registers, codes come from a bucket table over the
// L = 2^b - 1 decision points (up to 4096 buckets: finer grids separate the
// closer points of 63 levels).  A lane's eight codes make 8b bits of the row's
// little-endian bit stream; the four lanes of a quad hold 32 codes = b words,
// combined with quad broadcasts (DPP) and stored by the quad's lanes in turn.
// kErr: the row's error sums instead of the stored form, as in the 4-bit
// kernel, with the row table L[q] = bf16(G_q m) in the wave's LDS slot.
constexpr int kMaxBucketsN = 4096;

bool bucket_grid_n(const float* t, int L, BucketGrid& g) {
  uint32_t c[kMaxLevels];
  for (int j = 0; j < L; ++j) c[j] = float_bits(t[j]);
  if (c[0] <= 2 * kGuard) return false;
  for (int mbits = 3; mbits <= 12; ++mbits) {
    const int shift = 23 - mbits;
    const uint32_t b0 = (c[0] - kGuard) & ~((1u << shift) - 1u);
    const int64_t nb = (int64_t)((kTop - b0) >> shift) + 1;
    if (nb > kMaxBucketsN) return false;
    bool ok = true;
    for (int j = 0; j + 1 < L && ok; ++j)
      ok = ((c[j] + kGuard - b0) >> shift) < ((c[j + 1] - kGuard - b0) >> shift);
    if (ok) {
      g.b0 = b0;
      g.shift = shift;
      g.nb = (int)nb;
      g.size = table_slots(nb);
      return true;
    }
  }
  return false;
}

// The table of build_table over L points held in LDS.
__device__ void build_table_n(const float* pts, int L, BucketGrid g, uint2* tab) {
  for (int b = threadIdx.x; b < g.nb; b += blockDim.x) {
    const uint32_t lo = g.b0 + ((uint32_t)b << g.shift);
    const uint32_t hi = lo + (1u << g.shift);
    uint32_t below = 0u, next = kNoPoint;
    for (int j = L - 1; j >= 0; --j) {
      const uint32_t c = __float_as_uint(pts[j]);
      const bool under = c + kGuard < lo;
      below += under ? 1u : 0u;
      next = under ? next : c;
    }
    const uint32_t x = (next != kNoPoint && next - kGuard < hi) ? kGuard - next : kGuard - kNoPoint;
    tab[((g.b0 >> g.shift) + (uint32_t)b) & (uint32_t)(g.size - 1)] = make_uint2(x, below);
  }
}

// Word w of a 32-code block, the quad's fragments f[j] (8b bits each) laid
// end to end from bit 0.
template <int B>
__device__ __forceinline__ uint32_t block_word(const uint64_t (&f)[4], int w) {
  uint32_t out = 0u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int s = 8 * B * j - 32 * w;  // where fragment j starts relative to word w
    if (s >= 0 && s < 32) out |= (uint32_t)(f[j] << s);
    if (s < 0 && s > -8 * B) out |= (uint32_t)(f[j] >> (-s));
  }
  return out;
}

__device__ __forceinline__ uint32_t quad_bcast(uint32_t v, int j) {
  switch (j) {
    case 0: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x00, 0xF, 0xF, false);
    case 1: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x55, 0xF, 0xF, false);
    case 2: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xAA, 0xF, 0xF, false);
    default: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xFF, 0xF, 0xF, false);
  }
}

// Stores a lane's eight codes (q) and sign byte: the quad's 32 codes make b
// words at word index blk * b of the row; lane j of the quad stores words
// j and j + 4.  `valid` is uniform over a quad.
template <int B>
__device__ __forceinline__ void store_bits(uint32_t* prow, uint32_t* srow, int blk, int lane,
                                           bool valid, const uint32_t (&q)[8], uint32_t sbyte) {
  uint64_t frag = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) frag |= (uint64_t)q[i] << (B * i);
  uint64_t f[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    f[j] = (uint64_t)quad_bcast((uint32_t)frag, j) | ((uint64_t)quad_bcast((uint32_t)(frag >> 32), j) << 32);
  uint32_t s32 = valid ? (sbyte << (8 * (lane & 3))) : 0u;
  s32 |= (uint32_t)__builtin_amdgcn_mov_dpp((int)s32, 0xB1, 0xF, 0xF, false);
  s32 |= (uint32_t)__builtin_amdgcn_mov_dpp((int)s32, 0x4E, 0xF, 0xF, false);
  if (valid) {
    const int j = lane & 3;
#pragma unroll
    for (int w = 0; w < B; ++w)
      if ((w & 3) == j) store_stream(prow + blk * B + w, block_word<B>(f, w));
    if (j == 0) store_stream(srow + blk, s32);
  }
}

// The bucket table sits in dynamic LDS sized to the grid's slots (for
// alpha = 0.73: 52, 149 and 342 buckets for 3, 5 and 6 bits, in 64, 256 and
// 512 slots, against kMaxBucketsN),
// so the table does not cap the blocks per CU.  kOne as in quantize_block_rows.
extern __shared__ __attribute__((aligned(16))) unsigned char dyn_lds[];

template <typename T, int NCT, int B, bool kErr, bool kOne = false>
__global__ __launch_bounds__(kBlockThreads) void quantize_bits_rows(
    const T* __restrict__ w, int64_t n, int k, DecisionPointsN dp, BucketGrid g, LevelsN lv,
    uint32_t* __restrict__ packed, uint32_t* __restrict__ sign, float* __restrict__ scale,
    double* __restrict__ row_sums) {
  constexpr int L = (1 << B) - 1;
  constexpr int kWaves = kBlockThreads / kWave;
  uint2* s_tab = reinterpret_cast<uint2*>(dyn_lds);
  __shared__ float s_pts[kMaxLevels + 1];
  __shared__ double s_g[kMaxLevels + 1];
  __shared__ float s_wmax[2][kWaves];
  __shared__ uint32_t s_recw[kErr ? kWaves : 1][L + 1];
  __shared__ double s_sum[2][kWaves][2];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int64_t stride = gridDim.x;

  Slot<T> v[kOne ? 1 : 2][NCT];
  auto load_row = [&](int64_t rr, int buf) __attribute__((always_inline)) {
    const T* wr = w + rr * (int64_t)k;
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      const int e0 = c * kBlockChunk + tid * 8;
      if (e0 < k) v[buf][c].load_once(wr + e0); else v[buf][c].zero();
    }
  };
  int64_t row = blockIdx.x;
  if (row < n) load_row(row, 0);

  // decision points and levels to LDS (a lane-varying index into the argument
  // struct reads it from memory; this happens once per block)
  if (tid < L) s_pts[tid] = dp.t[tid];
  if (tid == L) s_pts[L] = 2.0f;
  if (kErr && tid <= L) s_g[tid] = lv.g[tid];
  lds_barrier();
  build_table_n(s_pts, L, g, s_tab);  // read after the first row-max barrier
  const int sh3 = g.shift - 3;
  const uint32_t mask8 = (uint32_t)(g.size - 1) << 3;
  const float ulo = __uint_as_float(g.b0);

  int64_t pend = -1;  // kErr: row whose partial sums wait in s_sum
  auto flush_sums = [&](int slot) __attribute__((always_inline)) {
    if (tid == 0 && pend >= 0) {
      double a0 = 0.0, a1 = 0.0;
#pragma unroll
      for (int q = 0; q < kWaves; ++q) {
        a0 += s_sum[slot][q][0];
        a1 += s_sum[slot][q][1];
      }
      row_sums[2 * pend] = a0;
      row_sums[2 * pend + 1] = a1;
    }
  };
  auto process = [&](int64_t rr, int buf, int ms) __attribute__((always_inline)) {
    typename Slot<T>::Acc acc = Slot<T>::acc0();
#pragma unroll
    for (int c = 0; c < NCT; ++c) v[buf][c].absmax(acc);
    float mx = wave_max(Slot<T>::finish(acc));
    if (lane == 0) s_wmax[ms][wave] = mx;
    lds_barrier();
    mx = s_wmax[ms][0];
#pragma unroll
    for (int q = 1; q < kBlockThreads / kWave; ++q) mx = fmaxf(mx, s_wmax[ms][q]);
    if constexpr (kErr) flush_sums(ms ^ 1);
    const bool fast = mx >= 0x1p-125f && mx <= 0x1p125f;
    const float r = 1.0f / mx;
    if constexpr (!kErr) {
      uint32_t* prow = packed + rr * (int64_t)(k / 32 * B);
      uint32_t* srow = sign + rr * (int64_t)(k / 32);
#pragma unroll
      for (int c = 0; c < NCT; ++c) {
        const int e0 = c * kBlockChunk + tid * 8;
        uint32_t q[8];
        codes8(v[buf][c], mx, r, fast, s_tab, sh3, mask8, ulo, s_pts, q);
        store_bits<B>(prow, srow, e0 >> 5, lane, e0 < k, q, sign_byte(v[buf][c]));
      }
      if (tid == 0) scale[rr] = mx;
    } else {
      if (lane <= L) s_recw[wave][lane] = bf16_rne_from_f64(s_g[lane] * (double)mx);
      wave_lds_sync();  // one wave's LDS ops complete in order
      float sw2 = 0.0f, se2 = 0.0f;
#pragma unroll
      for (int c = 0; c < NCT; ++c) {
        uint32_t q[8];
        codes8(v[buf][c], mx, r, fast, s_tab, sh3, mask8, ulo, s_pts, q);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float xv = v[buf][c].at(i);  // zero past k
          const float e = fabsf(xv) - __uint_as_float(s_recw[wave][q[i]] << 16);
          sw2 = fmaf(xv, xv, sw2);
          se2 = fmaf(e, e, se2);
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        sw2 += __shfl_xor(sw2, off, kWave);
        se2 += __shfl_xor(se2, off, kWave);
      }
      if (lane == 0) {
        s_sum[ms][wave][0] = sw2;
        s_sum[ms][wave][1] = se2;
      }
      pend = rr;
    }
  };

  if constexpr (kOne) {
    if (row < n) process(row, 0, 0);
  } else {
    while (row < n) {
      const int64_t r1 = row + stride;
      if (r1 < n) load_row(r1, 1);
      process(row, 0, 0);
      if (r1 >= n) break;
      const int64_t r2 = r1 + stride;
      if (r2 < n) load_row(r2, 0);
      process(r1, 1, 1);
      row = r2;
    }
  }
  if constexpr (kErr) {
    lds_barrier();
    const int64_t cnt = blockIdx.x < n ? (n - 1 - blockIdx.x) / stride + 1 : 0;
    flush_sums((int)((cnt - 1) & 1));
  }
}

// The codes of a row to a wave, as quantize_rows_table for four bits (rows of
// up to 2048 elements): the row (k <= NCH * 512) in the wave's registers, its
// max reduced across the wave with no block barrier, rows strided over at
// most kMaxRowBlocks blocks.  A lane holds elements c * 512 + 8 lane .. + 7 of
// chunk c, so the lanes of a quad hold 32 consecutive codes and store_bits
// packs them as the block kernel does.  The decision points and the bucket
// table are built in LDS once per block.
template <typename T, int NCH, int B>
__global__ __launch_bounds__(kRowsPerBlock * kWave) void quantize_bits_rows_table(
    const T* __restrict__ w, int64_t n, int k, DecisionPointsN dp, BucketGrid g,
    uint32_t* __restrict__ packed, uint32_t* __restrict__ sign, float* __restrict__ scale) {
  constexpr int L = (1 << B) - 1;
  uint2* s_tab = reinterpret_cast<uint2*>(dyn_lds);
  __shared__ float s_pts[kMaxLevels + 1];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int64_t stride = (int64_t)gridDim.x * kRowsPerBlock;
  int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + tid / kWave;

  // The first row's loads go out before the tables are built.
  Slot<T> v[NCH];
  auto load_row = [&](int64_t rr) __attribute__((always_inline)) {
    const T* wr = w + rr * (int64_t)k;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int e0 = c * kChunk + lane * 8;
      if (e0 < k) v[c].load_once(wr + e0); else v[c].zero();
    }
  };
  if (row < n) load_row(row);

  if (tid < L) s_pts[tid] = dp.t[tid];
  if (tid == L) s_pts[L] = 2.0f;
  lds_barrier();
  build_table_n(s_pts, L, g, s_tab);
  lds_barrier();  // the row loads stay in flight
  const int sh3 = g.shift - 3;
  const uint32_t mask8 = (uint32_t)(g.size - 1) << 3;
  const float ulo = __uint_as_float(g.b0);

  for (; row < n; row += stride) {
    typename Slot<T>::Acc acc = Slot<T>::acc0();
#pragma unroll
    for (int c = 0; c < NCH; ++c) v[c].absmax(acc);
    const float mx = wave_max(Slot<T>::finish(acc));
    const bool fast = mx >= 0x1p-125f && mx <= 0x1p125f;  // 1/m normal, u' <= 1 + ulps
    const float r = 1.0f / mx;
    uint32_t* prow = packed + row * (int64_t)(k / 32 * B);
    uint32_t* srow = sign + row * (int64_t)(k / 32);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int e0 = c * kChunk + lane * 8;
      uint32_t q[8];
      codes8(v[c], mx, r, fast, s_tab, sh3, mask8, ulo, s_pts, q);
      store_bits<B>(prow, srow, e0 >> 5, lane, e0 < k, q, sign_byte(v[c]));
    }
    if (lane == 0) scale[row] = mx;
    if (row + stride < n) load_row(row + stride);
  }
}

template <typename T, int NCH, int B>
hipError_t launch_bits_rows_table(const T* w, int64_t n, int64_t k, const DecisionPointsN& dp,
                                  const BucketGrid& g, uint32_t* packed, uint32_t* sign,
                                  float* scale, hipStream_t stream) {
  const int64_t groups = (n + kRowsPerBlock - 1) / kRowsPerBlock;
  const int64_t blocks = groups < kMaxRowBlocks ? groups : kMaxRowBlocks;
  hipLaunchKernelGGL((quantize_bits_rows_table<T, NCH, B>), dim3((unsigned)blocks),
                     dim3(kRowsPerBlock * kWave), (size_t)g.size * sizeof(uint2), stream, w, n,
                     (int)k, dp, g, packed, sign, scale);
  return hipGetLastError();
}

// Blocks of quantize_bits_rows<...> per CU with `dyn` bytes of table: computed
// once per kernel and KiB of table (the memo holds a count, so a race only
// computes it twice).
template <typename T, int NCT, int B, bool kErr, bool kOne>
int bits_blocks_per_cu(size_t dyn) {
  static std::atomic<int> memo[kMaxBucketsN * 8 / 1024 + 1];
  const size_t slot = (dyn + 1023) / 1024;
  int b = memo[slot].load(std::memory_order_relaxed);
  if (b == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, quantize_bits_rows<T, NCT, B, kErr, kOne>,
                                                     kBlockThreads, slot * 1024) != hipSuccess ||
        b < 1)
      b = 1;
    memo[slot].store(b, std::memory_order_relaxed);
  }
  return b;
}

template <typename T, int NCT, int B, bool kErr>
hipError_t launch_bits_rows(const T* w, int64_t n, int64_t k, const DecisionPointsN& dp,
                            const BucketGrid& g, const LevelsN& lv, uint32_t* packed,
                            uint32_t* sign, float* scale, double* row_sums, hipStream_t stream) {
  const size_t dyn = (size_t)g.size * sizeof(uint2);
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 1;
  // as launch_block_rows: twice the resident blocks, or a block per row
  if (n <= 2 * (int64_t)bits_blocks_per_cu<T, NCT, B, kErr, true>(dyn) * cus) {
    hipLaunchKernelGGL((quantize_bits_rows<T, NCT, B, kErr, true>), dim3((unsigned)n),
                       dim3(kBlockThreads), dyn, stream, w, n, (int)k, dp, g, lv, packed, sign,
                       scale, row_sums);
    return hipGetLastError();
  }
  const int64_t blocks = 2 * (int64_t)bits_blocks_per_cu<T, NCT, B, kErr, false>(dyn) * cus;
  hipLaunchKernelGGL((quantize_bits_rows<T, NCT, B, kErr>), dim3((unsigned)blocks),
                     dim3(kBlockThreads), dyn, stream, w, n, (int)k, dp, g, lv, packed, sign,
                     scale, row_sums);
  return hipGetLastError();
}

template <typename T, int B, bool kErr>
hipError_t dispatch_bits_nct(const T* w, int64_t n, int64_t k, const DecisionPointsN& dp,
                             const BucketGrid& g, const LevelsN& lv, uint32_t* packed,
                             uint32_t* sign, float* scale, double* row_sums, hipStream_t stream) {
  if constexpr (!kErr) {
    // Rows of up to 2048 elements: a row to a wave.  Side by side on one box
    // (graph replay, inputs past the Infinity Cache), 11520 x 1024 bfloat16:
    // 3 bits 18.0 -> 12.0 us, 5 bits 20.5 -> 14.3, 6 bits 25.4 -> 19.3.  Rows
    // of 3840 stay on the block kernel even with many rows, unlike the four-bit
    // codes: a wave per row measured 4-15 % slower on 11520 rows at every
    // width, and slower on 20480 rows at 3 and 5 bits.
    const int64_t nch = (k + kChunk - 1) / kChunk;
    if (nch <= 1) return launch_bits_rows_table<T, 1, B>(w, n, k, dp, g, packed, sign, scale, stream);
    if (nch <= 2) return launch_bits_rows_table<T, 2, B>(w, n, k, dp, g, packed, sign, scale, stream);
    if (nch <= 4) return launch_bits_rows_table<T, 4, B>(w, n, k, dp, g, packed, sign, scale, stream);
  }
  const int64_t nct = (k + kBlockChunk - 1) / kBlockChunk;
  if (nct <= 1)
    return launch_bits_rows<T, 1, B, kErr>(w, n, k, dp, g, lv, packed, sign, scale, row_sums, stream);
  if (nct <= 2)
    return launch_bits_rows<T, 2, B, kErr>(w, n, k, dp, g, lv, packed, sign, scale, row_sums, stream);
  if (nct <= 4)
    return launch_bits_rows<T, 4, B, kErr>(w, n, k, dp, g, lv, packed, sign, scale, row_sums, stream);
  return launch_bits_rows<T, 8, B, kErr>(w, n, k, dp, g, lv, packed, sign, scale, row_sums, stream);
}

template <typename T, bool kErr>
hipError_t dispatch_bits(const T* w, int64_t n, int64_t k, int bits, const DecisionPointsN& dp,
                         const LevelsN& lv, uint32_t* packed, uint32_t* sign, float* scale,
                         double* row_sums, hipStream_t stream) {
  BucketGrid g;
  if (!bucket_grid_n(dp.t, dp.n, g)) return hipErrorNotSupported;
  switch (bits) {
    case 3: return dispatch_bits_nct<T, 3, kErr>(w, n, k, dp, g, lv, packed, sign, scale, row_sums, stream);
    case 5: return dispatch_bits_nct<T, 5, kErr>(w, n, k, dp, g, lv, packed, sign, scale, row_sums, stream);
    case 6: return dispatch_bits_nct<T, 6, kErr>(w, n, k, dp, g, lv, packed, sign, scale, row_sums, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool error_sums_supported(const DecisionPoints& dp, int64_t k) {
  BucketGrid g;
  return bucket_grid(dp, g) && k <= 8 * kBlockChunk;
}

hipError_t launch_error_sums(const void* w, bool w_is_bf16, int64_t n, int64_t k,
                             const DecisionPoints& dp, const Levels& lv, double* row_sums,
                             hipStream_t stream) {
  if (w_is_bf16)
    return dispatch_error(static_cast<const uint16_t*>(w), n, k, dp, lv, row_sums, stream);
  return dispatch_error(static_cast<const float*>(w), n, k, dp, lv, row_sums, stream);
}

hipError_t launch_quantize(const void* w, bool w_is_bf16, int64_t n, int64_t k,
                           const DecisionPoints& dp, uint32_t* packed, uint32_t* sign,
                           float* scale, hipStream_t stream) {
  if (w_is_bf16)
    return dispatch(static_cast<const uint16_t*>(w), n, k, dp, packed, sign, scale, stream);
  return dispatch(static_cast<const float*>(w), n, k, dp, packed, sign, scale, stream);
}

bool bits_supported(const DecisionPointsN& dp, int64_t k) {
  BucketGrid g;
  return bucket_grid_n(dp.t, dp.n, g) && k <= 8 * kBlockChunk;
}

hipError_t launch_quantize_bits(const void* w, bool w_is_bf16, int64_t n, int64_t k, int bits,
                                const DecisionPointsN& dp, const LevelsN& lv, uint32_t* packed,
                                uint32_t* sign, float* scale, double* row_sums,
                                hipStream_t stream) {
  if (row_sums) {
    if (w_is_bf16)
      return dispatch_bits<uint16_t, true>(static_cast<const uint16_t*>(w), n, k, bits, dp, lv,
                                           nullptr, nullptr, nullptr, row_sums, stream);
    return dispatch_bits<float, true>(static_cast<const float*>(w), n, k, bits, dp, lv, nullptr,
                                      nullptr, nullptr, row_sums, stream);
  }
  if (w_is_bf16)
    return dispatch_bits<uint16_t, false>(static_cast<const uint16_t*>(w), n, k, bits, dp, lv,
                                          packed, sign, scale, nullptr, stream);
  return dispatch_bits<float, false>(static_cast<const float*>(w), n, k, bits, dp, lv, packed,
                                     sign, scale, nullptr, stream);
}

bool grouped_supported(const DecisionPoints& dp, const Levels& lv) {
  BucketGrid g;
  // every level times the smallest stored max (2^-24) stays a normal binary32
  return bucket_grid(dp, g) && lv.g[1] * 0x1p-24 >= 0x1p-126;
}

hipError_t launch_quantize_grouped(const void* w, bool w_is_bf16, int64_t n, int64_t k, int gs,
                                   const DecisionPoints& dp, uint32_t* packed, uint32_t* sign,
                                   uint16_t* scale16, hipStream_t stream) {
  if (w_is_bf16)
    return dispatch_grouped(static_cast<const uint16_t*>(w), n, k, gs, dp, packed, sign, scale16,
                            stream);
  return dispatch_grouped(static_cast<const float*>(w), n, k, gs, dp, packed, sign, scale16,
                          stream);
}

}  // namespace opq
