// OPQ dequantize kernel (model card "OPQ INT4 Z-Image", section
// "技术细节 / 推理解码"): w' = sign * (q/15)^(1/alpha) * m, stored as bfloat16.
//
// The power is never evaluated per element: each row has a sixteen-entry
// table L[q] = bf16(G_q * m) with G_q = (q/15)^(1/alpha) from the host, rounded
// once from double.  Lanes 0..15 of the wave compute one entry each; the table
// is then held as byte planes in registers and looked up with v_perm_b32
// (decode.hpp).  Code 0 gives +0.0 whatever the sign bit.
//
// One wave per row.  A lane turns one packed word (eight codes) and a byte of
// the sign plane into 16 bytes of bfloat16 per 512-element chunk; the loads of
// up to kGroup chunks are issued before any of them is decoded.  HBM traffic
// is the algorithmic 0.625 B read + 2 B written per weight.
#include "decode.hpp"
#include "device_common.hpp"
#include "group.hpp"

namespace opq {
namespace {

constexpr int kRowsPerBlock = 4;
constexpr int kChunk = kWave * 8;
constexpr int kGroup = 8;  // chunks whose loads are in flight together

__global__ __launch_bounds__(kRowsPerBlock * kWave) void dequantize_rows(
    const uint32_t* __restrict__ packed, const uint32_t* __restrict__ sign,
    const float* __restrict__ scale, int64_t n, int k, Levels lv, uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x / kWave);
  if (row >= n) return;  // whole waves leave; no block-wide barrier
  const uint32_t* prow = packed + row * (int64_t)(k / 8);
  const uint32_t* srow = sign + row * (int64_t)(k / 32);
  uint16_t* orow = out + row * (int64_t)k;
  const int nch = (k + kChunk - 1) / kChunk;

  RowLut t;
  for (int c0 = 0; c0 < nch; c0 += kGroup) {
    uint32_t wv[kGroup], sv[kGroup];
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      const int e0 = (c0 + g) * kChunk + lane * 8;
      const bool valid = e0 < k;
      wv[g] = valid ? prow[e0 / 8] : 0u;
      sv[g] = valid ? srow[e0 / 32] : 0u;
    }
    if (c0 == 0) {
      // while the first loads are in flight: lane q makes L[q]
      const uint32_t e = lut_entry(lv, lane & 15, scale[row]);
      t = row_lut_from_lanes(e);
    }
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      const int e0 = (c0 + g) * kChunk + lane * 8;
      if (e0 < k) {
        uint32_t o[4];
        decode_word_ordered(wv[g], sv[g] >> (8 * (lane & 3)), t, o);
        *reinterpret_cast<uint4*>(orow + e0) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
  }
}

// Group-wise form.  The codes stream as one flat array; a lane decodes
// kGWords consecutive packed words (8 kGWords codes, which lie in one group)
// per chunk: it makes that group's table itself (make_row_lut with the
// float16 max, the code index uniform so the levels stay in scalar
// registers), then moves 4 kGWords bytes of codes and 16 kGWords of bf16.
// Each wave takes kGUnroll chunks with all their loads in flight; there is no
// LDS and no barrier, so the grid is simply one wave per kGUnroll chunks.
constexpr int kGThreads = 256;
constexpr int kGUnroll = 2;
constexpr int kGWords = 2;                   // packed words per lane per chunk
constexpr int kGChunk = kWave * 8 * kGWords;  // elements per wave per chunk

template <int GS>
__global__ __launch_bounds__(kGThreads) void dequantize_grouped_rows(
    const uint32_t* __restrict__ packed, const uint32_t* __restrict__ sign,
    const uint16_t* __restrict__ scale16, int64_t total, Levels lv, uint16_t* __restrict__ out) {
  static_assert(GS % (8 * kGWords) == 0, "a lane's codes lie in one group");
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
#pragma unroll
  for (int u = 0; u < kGUnroll; ++u) {
    const int64_t e0 = (wid * kGUnroll + u) * kGChunk + lane * 8 * kGWords;
    if (e0 < total) {
      const RowLut t = make_row_lut(lv, f16_value(hv[u]));
#pragma unroll
      for (int j = 0; j < kGWords; ++j) {
        uint32_t o[4];
        decode_word_ordered(wv[u][j], sv[u] >> (8 * j), t, o);
        *reinterpret_cast<uint4*>(out + e0 + 8 * j) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
  }
}

template <int GS>
hipError_t launch_grouped(const uint32_t* packed, const uint32_t* sign, const uint16_t* scale16,
                          int64_t total, const Levels& lv, uint16_t* out, hipStream_t stream) {
  const int64_t per_block = (int64_t)kGChunk * kGUnroll * (kGThreads / kWave);
  const int64_t blocks = (total + per_block - 1) / per_block;
  hipLaunchKernelGGL((dequantize_grouped_rows<GS>), dim3((unsigned)blocks), dim3(kGThreads), 0,
                     stream, packed, sign, scale16, total, lv, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dequantize_grouped(const uint32_t* packed, const uint32_t* sign,
                                     const uint16_t* scale16, int64_t n, int64_t k, int gs,
                                     const Levels& lv, uint16_t* out, hipStream_t stream) {
  const int64_t total = n * k;
  switch (gs) {
    case 32: return launch_grouped<32>(packed, sign, scale16, total, lv, out, stream);
    case 64: return launch_grouped<64>(packed, sign, scale16, total, lv, out, stream);
    case 128: return launch_grouped<128>(packed, sign, scale16, total, lv, out, stream);
    case 256: return launch_grouped<256>(packed, sign, scale16, total, lv, out, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_dequantize(const uint32_t* packed, const uint32_t* sign, const float* scale,
                             int64_t n, int64_t k, const Levels& lv, uint16_t* out,
                             hipStream_t stream) {
  const int64_t blocks = (n + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL(dequantize_rows, dim3((unsigned)blocks), dim3(kRowsPerBlock * kWave), 0,
                     stream, packed, sign, scale, n, (int)k, lv, out);
  return hipGetLastError();
}

}  // namespace opq
