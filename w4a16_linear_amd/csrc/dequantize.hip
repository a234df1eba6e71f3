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

#include <algorithm>

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

// Group-wise form.  The codes stream as one flat array: a lane decodes one
// packed word (eight codes of one group) per 512-element chunk, kGUnroll
// chunks' loads in flight.  Each block first writes the 1024 x 16 table of
// bf16(G_q (1 + mt/1024)) to LDS (group.hpp, while its first loads are in
// flight); a lane's group table is then one table row with the group max's
// exponent added, held as byte planes for the v_perm decoder.
constexpr int kGThreads = 256;
constexpr int kGUnroll = 4;

template <int GS>
__global__ __launch_bounds__(kGThreads) void dequantize_grouped_rows(
    const uint32_t* __restrict__ packed, const uint32_t* __restrict__ sign,
    const uint16_t* __restrict__ scale16, int64_t total, Levels lv, uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint32_t s_mt[kMantissas * 8];
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t nchunks = (total + kChunk - 1) / kChunk;
  const int64_t wid = (int64_t)blockIdx.x * (kGThreads / kWave) + threadIdx.x / kWave;
  const int64_t step = (int64_t)gridDim.x * (kGThreads / kWave) * kGUnroll;

  uint32_t wv[kGUnroll], sv[kGUnroll], hv[kGUnroll];
  auto load = [&](int64_t cb) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kGUnroll; ++u) {
      const int64_t e0 = (cb + u) * kChunk + lane * 8;
      const bool valid = e0 < total;
      wv[u] = valid ? packed[e0 >> 3] : 0u;
      sv[u] = valid ? sign[e0 >> 5] : 0u;
      hv[u] = valid ? scale16[e0 / GS] : 0u;
    }
  };
  int64_t cb = wid * kGUnroll;
  if (cb < nchunks) load(cb);
  build_mant_table(lv, s_mt);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the table is written
  __builtin_amdgcn_s_barrier();

  for (; cb < nchunks; cb += step) {
    uint32_t o[kGUnroll][4];
#pragma unroll
    for (int u = 0; u < kGUnroll; ++u)
      decode_word_ordered(wv[u], sv[u] >> (8 * (lane & 3)), group_lut(s_mt, hv[u]), o[u]);
    const int64_t c0 = cb;
    if (cb + step < nchunks) load(cb + step);  // the next batch goes out before the stores
#pragma unroll
    for (int u = 0; u < kGUnroll; ++u) {
      const int64_t e0 = (c0 + u) * kChunk + lane * 8;
      if (e0 < total)
        *reinterpret_cast<uint4*>(out + e0) = make_uint4(o[u][0], o[u][1], o[u][2], o[u][3]);
    }
  }
}

template <int GS>
hipError_t launch_grouped(const uint32_t* packed, const uint32_t* sign, const uint16_t* scale16,
                          int64_t total, const Levels& lv, uint16_t* out, hipStream_t stream) {
  static const int per_cu = [] {
    int b = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b, dequantize_grouped_rows<GS>, kGThreads,
                                                     0) != hipSuccess || b < 1)
      b = 1;
    return b;
  }();
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 1;
  const int64_t batches = (total + (int64_t)kChunk * kGUnroll - 1) / ((int64_t)kChunk * kGUnroll);
  const int64_t blocks = std::min<int64_t>((int64_t)per_cu * cus,
                                           (batches + kGThreads / kWave - 1) / (kGThreads / kWave));
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
