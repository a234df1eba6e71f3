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

}  // namespace

hipError_t launch_dequantize(const uint32_t* packed, const uint32_t* sign, const float* scale,
                             int64_t n, int64_t k, const Levels& lv, uint16_t* out,
                             hipStream_t stream) {
  const int64_t blocks = (n + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL(dequantize_rows, dim3((unsigned)blocks), dim3(kRowsPerBlock * kWave), 0,
                     stream, packed, sign, scale, n, (int)k, lv, out);
  return hipGetLastError();
}

}  // namespace opq
