// OPQ dequantize kernel (model card "OPQ INT4 Z-Image", section
// "技术细节 / 推理解码"): w' = sign * (q/15)^(1/alpha) * m, stored as bfloat16.
//
// The power is never evaluated per element: each row has a sixteen-entry
// table L[q] = bf16(G_q * m) with G_q = (q/15)^(1/alpha) from the host, rounded
// once from double.  Lanes 0..15 of the wave hold the table; every lane looks
// its codes up with a cross-lane read.  Code 0 gives +0.0 whatever the sign.
//
// One wave per row; each lane turns one packed word (eight codes) and a byte of
// the sign plane into 16 bytes of bfloat16 per step.  HBM traffic is the
// algorithmic 0.625 B read + 2 B written per weight.
#include "device_common.hpp"

namespace opq {
namespace {

constexpr int kRowsPerBlock = 4;
constexpr int kChunk = kWave * 8;

__global__ __launch_bounds__(kRowsPerBlock * kWave) void dequantize_rows(
    const uint32_t* __restrict__ packed, const uint32_t* __restrict__ sign,
    const float* __restrict__ scale, int64_t n, int k, Levels lv, uint16_t* __restrict__ out) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x / kWave);
  if (row >= n) return;
  const float m = scale[row];
  const uint32_t lut = lut_entry(lv, lane & 15, m);  // lane q holds L[q]
  const uint32_t* prow = packed + row * (int64_t)(k / 8);
  const uint32_t* srow = sign + row * (int64_t)(k / 32);
  uint16_t* orow = out + row * (int64_t)k;
  const int nch = (k + kChunk - 1) / kChunk;
  for (int c = 0; c < nch; ++c) {  // uniform trip count: every lane joins the shuffles
    const int e0 = c * kChunk + lane * 8;
    const bool valid = e0 < k;
    const uint32_t word = valid ? prow[e0 / 8] : 0u;
    const uint32_t sbyte = valid ? (srow[e0 / 32] >> (e0 & 31)) & 0xFFu : 0u;
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = (word >> (4 * i)) & 15;
      uint32_t h = (uint32_t)__shfl((int)lut, q, kWave);
      if (q != 0 && ((sbyte >> i) & 1u)) h |= 0x8000u;
      if (i & 1) o[i >> 1] |= h << 16;
      else o[i >> 1] = h;
    }
    if (valid) *reinterpret_cast<uint4*>(orow + e0) = make_uint4(o[0], o[1], o[2], o[3]);
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
