// OPQ dequantize kernel (model card "OPQ INT4 Z-Image", section
// "技术细节 / 推理解码"): w' = sign * (q/15)^(1/alpha) * m, stored as bfloat16.
//
// The power is never evaluated per element: each row has a sixteen-entry
// table L[q] = bf16(G_q * m) with G_q = (q/15)^(1/alpha) from the host, rounded
// once from double.  Lanes 0..15 of the wave compute one entry each; the table
// is then held as byte planes in registers and looked up with v_perm_b32
// (decode.hpp).  Code 0 gives +0.0 whatever the sign bit.
//
// One wave per row segment of up to kRowGroup 512-element chunks (a row of
// k = 10240 is five segments), so every wave has all its loads in flight at
// once and long rows still give many waves.  A lane turns one packed word
// (eight codes) and a byte of the sign plane into 16 bytes of bfloat16 per
// chunk; each wave makes its row's table.  HBM traffic is the algorithmic
// 0.625 B read + 2 B written per weight.  The bfloat16 output is a one-touch
// stream and is stored nontemporal (8 % faster on large layers, 20 % on a
// 3840 x 3840 weight, than plain stores).
//
// Further down: the group-wise form (one float16 max per group of weights)
// and 3/5/6-bit codes.
#include <algorithm>

#include "decode.hpp"
#include "device_common.hpp"
#include "group.hpp"

namespace opq {
namespace {

constexpr int kRowsPerBlock = 4;
constexpr int kChunk = kWave * 8;
constexpr int kGroup = 8;  // chunks whose loads are in flight together (b-bit codes)
// The same for the 4-bit codes: segments of 4 chunks instead of 8 made
// dequantize 3-4 % faster on the DiT layers (20480 x 3840 37.9 -> 36.8 us,
// 11520 x 3840 23.7 -> 22.7 us, 3840 x 10240 21.5 -> 20.5 us; 3840 x 3840
// equal; inputs past the Infinity Cache, variants interleaved on one box);
// 2 chunks, 8 waves per block and nontemporal loads were slower.
constexpr int kRowGroup = 4;

// segs = segments per row (ceil(chunks / kRowGroup)); wave w of block b takes
// segment (4b + w) % segs of row (4b + w) / segs.
__global__ __launch_bounds__(kRowsPerBlock * kWave) void dequantize_rows(
    const uint32_t* __restrict__ packed, const uint32_t* __restrict__ sign,
    const float* __restrict__ scale, int64_t n, int k, int segs, Levels lv,
    uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t unit = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x / kWave);
  const int64_t row = unit / segs;
  if (row >= n) return;  // whole waves leave; no block-wide barrier
  const int c0 = (int)(unit - row * segs) * kRowGroup;  // first chunk of the segment
  const uint32_t* prow = packed + row * (int64_t)(k / 8);
  const uint32_t* srow = sign + row * (int64_t)(k / 32);
  uint16_t* orow = out + row * (int64_t)k;

  uint32_t wv[kRowGroup], sv[kRowGroup];
#pragma unroll
  for (int g = 0; g < kRowGroup; ++g) {
    const int e0 = (c0 + g) * kChunk + lane * 8;
    const bool valid = e0 < k;
    wv[g] = valid ? prow[e0 / 8] : 0u;
    sv[g] = valid ? srow[e0 / 32] : 0u;
  }
  // while the loads are in flight: lane q makes L[q]
  const RowLut t = row_lut_from_lanes(lut_entry(lv, lane & 15, scale[row]));
#pragma unroll
  for (int g = 0; g < kRowGroup; ++g) {
    const int e0 = (c0 + g) * kChunk + lane * 8;
    if (e0 < k) {
      uint32_t o[4];
      decode_word_ordered(wv[g], sv[g] >> (8 * (lane & 3)), t, o);
      store_stream16(orow + e0, o[0], o[1], o[2], o[3]);
    }
  }
}

// Group-wise form.  The codes stream as one flat array; a lane decodes
// kGWords consecutive packed words (8 kGWords codes, which lie in one group)
// per chunk and moves 4 kGWords bytes of codes and 16 kGWords of bf16.  The
// group's table bf16(G_q m16) is made by the group's lanes together: with
// LG = GS / (8 kGWords) lanes per group, each makes 16 / LG entries (at least
// a pair) from the levels in LDS, and the eight pair words are then gathered
// to every lane of the group with ds_bpermute and cut into byte planes.  Each
// wave takes kGUnroll chunks with all their loads in flight; the grid is one
// wave per kGUnroll chunks.
//
// One word per lane, so each store instruction of a wave writes 1 KB of
// consecutive bf16 and the stores can go nontemporal: with two words per lane
// (32 bytes per lane, written by two 16-byte stores that each cover every
// other 16 bytes) nontemporal stores took 51 us for a 11520 x 3840 weight in
// groups of 128, plain ones 31 us, and this layout 27 us, although it makes a
// table per 8 codes instead of per 16.
constexpr int kGThreads = 256;
constexpr int kGUnroll = 4;
constexpr int kGWords = 1;                    // packed words per lane per chunk
constexpr int kGChunk = kWave * 8 * kGWords;  // elements per wave per chunk

// Byte planes of the table of this lane's group: the group spans LG lanes
// from `base`, its stored max is m16 (the same in all of them).
template <int LG>
__device__ __forceinline__ RowLut group_lut_shared(const double* s_g, float m16, int lane) {
  constexpr int D = (16 / LG) / 2 > 0 ? (16 / LG) / 2 : 1;  // pair words per lane
  constexpr int H = 8 / D;                                // lanes holding distinct words
  const int j = lane % LG, base = lane - j;
  const int slot = j % H;
  const double m = (double)m16;
  uint32_t mine[D];
#pragma unroll
  for (int i = 0; i < D; ++i) {
    const int q = 2 * (D * slot + i);
    mine[i] = bf16_rne_from_f64(s_g[q] * m) | (bf16_rne_from_f64(s_g[q + 1] * m) << 16);
  }
  uint32_t d[8];
#pragma unroll
  for (int w = 0; w < 8; ++w)
    d[w] = (uint32_t)__builtin_amdgcn_ds_bpermute((base + w / D) * 4, (int)mine[w % D]);
  RowLut t;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    t.lo[i] = __builtin_amdgcn_perm(d[2 * i + 1], d[2 * i], 0x06040200u);
    t.hi[i] = __builtin_amdgcn_perm(d[2 * i + 1], d[2 * i], 0x07050301u);
  }
  return t;
}

template <int GS>
__global__ __launch_bounds__(kGThreads) void dequantize_grouped_rows(
    const uint32_t* __restrict__ packed, const uint32_t* __restrict__ sign,
    const uint16_t* __restrict__ scale16, int64_t total, Levels lv, uint16_t* __restrict__ out) {
  static_assert(GS % (8 * kGWords) == 0, "a lane's codes lie in one group");
  constexpr int LG = GS / (8 * kGWords);  // lanes per group
  __shared__ double s_g[kLevels + 1];
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wid = (int64_t)blockIdx.x * (kGThreads / kWave) + threadIdx.x / kWave;
  uint32_t wv[kGUnroll][kGWords], sv[kGUnroll], hv[kGUnroll];
#pragma unroll
  for (int u = 0; u < kGUnroll; ++u) {
    const int64_t e0 = (wid * kGUnroll + u) * kGChunk + lane * 8 * kGWords;
    const bool valid = e0 < total;
    if constexpr (kGWords == 4) {
      const uint4 v = valid ? *reinterpret_cast<const uint4*>(packed + (e0 >> 3)) : make_uint4(0, 0, 0, 0);
      wv[u][0] = v.x; wv[u][1] = v.y; wv[u][2] = v.z; wv[u][3] = v.w;
    } else if constexpr (kGWords == 2) {
      const uint2 v = valid ? *reinterpret_cast<const uint2*>(packed + (e0 >> 3)) : make_uint2(0, 0);
      wv[u][0] = v.x; wv[u][1] = v.y;
    } else {
      wv[u][0] = valid ? packed[e0 >> 3] : 0u;
    }
    sv[u] = valid ? sign[e0 >> 5] >> (kGWords == 4 ? 0 : 8 * ((e0 >> 3) & 3)) : 0u;
    hv[u] = valid ? scale16[e0 / GS] : 0u;
  }
  if (threadIdx.x <= kLevels) s_g[threadIdx.x] = lv.g[threadIdx.x];
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kGUnroll; ++u) {
    const int64_t e0 = (wid * kGUnroll + u) * kGChunk + lane * 8 * kGWords;
    // every lane takes part in the gathers, valid or not
    const RowLut t = group_lut_shared<LG>(s_g, f16_value(hv[u]), lane);
    if (e0 < total) {
#pragma unroll
      for (int j = 0; j < kGWords; ++j) {
        uint32_t o[4];
        decode_word_ordered(wv[u][j], sv[u] >> (8 * j), t, o);
        store_stream16(out + e0 + 8 * j, o[0], o[1], o[2], o[3]);
      }
    }
  }
}

template <int GS>
hipError_t launch_grouped(const uint32_t* packed, const uint32_t* sign, const uint16_t* scale16,
                          int64_t n, int64_t k, const Levels& lv, uint16_t* out,
                          hipStream_t stream) {
  const int64_t per_block = (int64_t)kGChunk * kGUnroll * (kGThreads / kWave);
  const int64_t per_thread = per_block / kGThreads;
  const int64_t max_rows = std::max<int64_t>(1, kMaxLaunchThreads * per_thread / k);
  for (int64_t r0 = 0; r0 < n; r0 += max_rows) {  // groups never straddle rows
    const int64_t total = std::min(max_rows, n - r0) * k;
    const int64_t blocks = (total + per_block - 1) / per_block;
    hipLaunchKernelGGL((dequantize_grouped_rows<GS>), dim3((unsigned)blocks), dim3(kGThreads), 0,
                       stream, packed + r0 * (k / 8), sign + r0 * (k / 32),
                       scale16 + r0 * (k / GS), total, lv, out + r0 * k);
  }
  return hipGetLastError();
}

// b-bit codes (3, 5 or 6 bits; 2^b - 1 levels).  One wave per row segment as
// in dequantize_rows; the row's table L[q] = bf16(G_q m), q = 0 .. 2^b - 1, sits
// in the wave's LDS slot (lane q makes entry q from the levels, which the block
// copies to LDS once).  A lane decodes eight codes per 512-element chunk: its
// 8b bits of the row's bit stream start at bit 8b (lane + 64 c), a multiple of
// 8 below 32 within their word, so they lie in two consecutive words.
// kStream: the output is the caller's (nontemporal stores, as dequantize_rows);
// otherwise it is W' for the dense linear kernel that runs next, and plain
// stores leave it in cache for that kernel (nontemporal ones made the b-bit
// linear layer 4-13 % slower).
template <int B, bool kStream>
__global__ __launch_bounds__(kRowsPerBlock * kWave) void dequantize_bits_rows(
    const uint32_t* __restrict__ packed, const uint32_t* __restrict__ sign,
    const float* __restrict__ scale, int64_t n, int k, int segs, LevelsN lv,
    uint16_t* __restrict__ out) {
  constexpr int L = (1 << B) - 1;
  __shared__ double s_g[L + 1];
  __shared__ uint32_t s_lut[kRowsPerBlock][L + 1];
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  if (threadIdx.x <= L) s_g[threadIdx.x] = lv.g[threadIdx.x];
  __syncthreads();  // every wave passes here before any leaves
  const int64_t unit = (int64_t)blockIdx.x * kRowsPerBlock + wave;  // row segment, as in dequantize_rows
  const int64_t row = unit / segs;
  if (row >= n) return;
  const int c0 = (int)(unit - row * segs) * kGroup;
  if (lane <= L) s_lut[wave][lane] = bf16_rne_from_f64(s_g[lane] * (double)scale[row]);
  wave_lds_sync();  // one wave's LDS ops complete in order
  const int nwords = k / 32 * B;
  const uint32_t* prow = packed + row * (int64_t)nwords;
  const uint32_t* srow = sign + row * (int64_t)(k / 32);
  uint16_t* orow = out + row * (int64_t)k;
  uint32_t w0[kGroup], w1[kGroup], sv[kGroup];
#pragma unroll
  for (int g = 0; g < kGroup; ++g) {
    const int e0 = (c0 + g) * kChunk + lane * 8;
    const bool valid = e0 < k;
    const int wi = (e0 * B) >> 5;
    w0[g] = valid ? prow[wi] : 0u;
    w1[g] = valid ? prow[min(wi + 1, nwords - 1)] : 0u;  // past the row only when unused
    sv[g] = valid ? srow[e0 / 32] : 0u;
  }
#pragma unroll
  for (int g = 0; g < kGroup; ++g) {
    const int e0 = (c0 + g) * kChunk + lane * 8;
    if (e0 < k) {
      const uint64_t f = (((uint64_t)w1[g] << 32) | w0[g]) >> ((e0 * B) & 31);
      const uint32_t sb = sv[g] >> (8 * (lane & 3));
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const uint32_t q0 = (uint32_t)(f >> (B * i)) & L, q1 = (uint32_t)(f >> (B * (i + 1))) & L;
        uint32_t v0 = s_lut[wave][q0], v1 = s_lut[wave][q1];
        if (((sb >> i) & 1u) && q0) v0 |= 0x8000u;
        if (((sb >> (i + 1)) & 1u) && q1) v1 |= 0x8000u;
        o[i / 2] = v0 | (v1 << 16);
      }
      if constexpr (kStream)
        store_stream16(orow + e0, o[0], o[1], o[2], o[3]);
      else
        *reinterpret_cast<uint4*>(orow + e0) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

template <int B>
void launch_bits_rows(dim3 grid, dim3 block, hipStream_t stream, bool stream_out,
                      const uint32_t* p, const uint32_t* sg, const float* sc, int64_t nr, int k,
                      int segs, const LevelsN& lv, uint16_t* o) {
  if (stream_out)
    hipLaunchKernelGGL((dequantize_bits_rows<B, true>), grid, block, 0, stream, p, sg, sc, nr, k, segs, lv, o);
  else
    hipLaunchKernelGGL((dequantize_bits_rows<B, false>), grid, block, 0, stream, p, sg, sc, nr, k, segs, lv, o);
}

}  // namespace

hipError_t launch_dequantize_bits(const uint32_t* packed, const uint32_t* sign,
                                  const float* scale, int64_t n, int64_t k, int bits,
                                  const LevelsN& lv, uint16_t* out, bool stream_out,
                                  hipStream_t stream) {
  if (bits != 3 && bits != 5 && bits != 6) return hipErrorInvalidValue;
  const int64_t nch = (k + kChunk - 1) / kChunk;
  const int segs = (int)(nch > 0 ? (nch + kGroup - 1) / kGroup : 1);
  const int64_t max_rows = kMaxLaunchThreads / kWave / segs;  // a wave per row segment
  for (int64_t r0 = 0; r0 < n; r0 += max_rows) {
    const int64_t nr = std::min(max_rows, n - r0);
    const int64_t blocks = (nr * segs + kRowsPerBlock - 1) / kRowsPerBlock;
    const uint32_t* p = packed + r0 * (k * bits / 32);
    const uint32_t* sg = sign + r0 * (k / 32);
    const float* sc = scale + r0;
    uint16_t* o = out + r0 * k;
    const dim3 grid((unsigned)blocks), block(kRowsPerBlock * kWave);
    if (bits == 3)
      launch_bits_rows<3>(grid, block, stream, stream_out, p, sg, sc, nr, (int)k, segs, lv, o);
    else if (bits == 5)
      launch_bits_rows<5>(grid, block, stream, stream_out, p, sg, sc, nr, (int)k, segs, lv, o);
    else
      launch_bits_rows<6>(grid, block, stream, stream_out, p, sg, sc, nr, (int)k, segs, lv, o);
  }
  return hipGetLastError();
}

hipError_t launch_dequantize_grouped(const uint32_t* packed, const uint32_t* sign,
                                     const uint16_t* scale16, int64_t n, int64_t k, int gs,
                                     const Levels& lv, uint16_t* out, hipStream_t stream) {
  switch (gs) {
    case 32: return launch_grouped<32>(packed, sign, scale16, n, k, lv, out, stream);
    case 64: return launch_grouped<64>(packed, sign, scale16, n, k, lv, out, stream);
    case 128: return launch_grouped<128>(packed, sign, scale16, n, k, lv, out, stream);
    case 256: return launch_grouped<256>(packed, sign, scale16, n, k, lv, out, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_dequantize(const uint32_t* packed, const uint32_t* sign, const float* scale,
                             int64_t n, int64_t k, const Levels& lv, uint16_t* out,
                             hipStream_t stream) {
  const int64_t nch = (k + kChunk - 1) / kChunk;
  const int64_t segs = nch > 0 ? (nch + kRowGroup - 1) / kRowGroup : 1;
  const int64_t max_rows = kMaxLaunchThreads / kWave / segs;  // a wave per segment
  for (int64_t r0 = 0; r0 < n; r0 += max_rows) {
    const int64_t nr = std::min(max_rows, n - r0);
    const int64_t blocks = (nr * segs + kRowsPerBlock - 1) / kRowsPerBlock;
    hipLaunchKernelGGL(dequantize_rows, dim3((unsigned)blocks), dim3(kRowsPerBlock * kWave), 0,
                       stream, packed + r0 * (k / 8), sign + r0 * (k / 32), scale + r0, nr,
                       (int)k, (int)segs, lv, out + r0 * k);
  }
  return hipGetLastError();
}

}  // namespace opq
