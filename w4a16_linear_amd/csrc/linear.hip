// OPQ W4A16 linear layer: y = x W'^T (+ bias), with W' the bfloat16
// reconstruction of the stored weights (model card "OPQ INT4 Z-Image": the
// OPQLinear layer of the file list, decoded as in "技术细节 / 推理解码").
//
// W' is never written to HBM.  Each block builds the sixteen-entry table
// L_n[q] = bf16(G_q * m_n) for its weight rows in LDS, turns packed codes and
// sign bits into bfloat16 on chip, and feeds bf16 MFMA with fp32 accumulation.
// The table holds the same values opq_dequantize writes; the scale is never
// applied after the product.
//
// Two paths:
//  * m <= kSkinnyMaxM: weight-streaming (HBM-bound).  A block owns 16 weight
//    rows and all of k; its waves split k and reduce through LDS.  W' is the
//    A operand of v_mfma_f32_16x16x32_bf16 (one packed word = a lane's eight
//    k values), x^T the B operand.
//  * otherwise: 128x128 output tiles, k steps of 64, x and dequantized W'
//    staged through LDS, 2x2 waves each on 64x64 with v_mfma_f32_32x32x16_bf16.
#include "device_common.hpp"

namespace opq {
namespace {

// ---------------------------------------------------------------- skinny path

constexpr int kSkinnyMaxM = 64;
constexpr int kSkRows = 16;    // weight rows per block
constexpr int kSkWaves = 8;    // waves splitting k

__global__ __launch_bounds__(kSkWaves * kWave) void linear_skinny(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ packed,
    const uint32_t* __restrict__ sign, const float* __restrict__ scale,
    const float* __restrict__ bias, int m, int n, int k, Levels lv, float* __restrict__ y) {
  __shared__ uint16_t s_lut[kSkRows * 16];
  __shared__ float s_red[kSkWaves][4][4][kWave];  // wave, m-block, acc reg, lane

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int n0 = blockIdx.x * kSkRows;

  if (tid < kSkRows * 16) {
    const int r = tid >> 4, q = tid & 15;
    const int gn = n0 + r;
    s_lut[tid] = (uint16_t)lut_entry(lv, q, gn < n ? scale[gn] : 0.0f);
  }
  __syncthreads();

  const int nmb = (m + 15) / 16;  // 16-row blocks of x, at most 4
  const int r = lane & 15;        // weight row of this lane's A fragment
  const int g = lane >> 4;        // which eight k of the 32-wide step
  const int gn = n0 + r;
  const int kwords = k / 8, swords = k / 32;
  const uint16_t* lut = s_lut + r * 16;

  floatx4_t acc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) acc[b] = floatx4_t{0.f, 0.f, 0.f, 0.f};

  for (int s = wave; s < swords; s += kSkWaves) {
    const int kb = s * 32 + 8 * g;
    uint32_t wd = 0u, sw = 0u;
    if (gn < n) {
      wd = packed[(int64_t)gn * kwords + kb / 8];
      sw = sign[(int64_t)gn * swords + s];
    }
    const uint32_t sbyte = (sw >> (8 * g)) & 0xFFu;
    uint32_t w4[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t h = lut[(wd >> (4 * i)) & 15u];
      h |= ((sbyte >> i) & 1u) << 15;
      if (i & 1) w4[i >> 1] |= h << 16;
      else w4[i >> 1] = h;
    }
    const bf16x8_t a = __builtin_bit_cast(bf16x8_t, make_uint4(w4[0], w4[1], w4[2], w4[3]));
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (b < nmb) {
        const int mm = b * 16 + r;
        uint4 xv = make_uint4(0u, 0u, 0u, 0u);
        if (mm < m) xv = *reinterpret_cast<const uint4*>(x + (int64_t)mm * k + kb);
        acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8_t, xv),
                                                         acc[b], 0, 0, 0);
      }
    }
  }

#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int j = 0; j < 4; ++j) s_red[wave][b][j][lane] = acc[b][j];
  __syncthreads();

  // Output (mm, row i of the block): fragment element D[i][mm % 16] of block
  // mm / 16 sits in lane 16 * (i / 4) + mm % 16, register i % 4.
  for (int o = tid; o < kSkRows * nmb * 16; o += kSkWaves * kWave) {
    const int i = o % kSkRows;
    const int mm = o / kSkRows;
    const int b = mm / 16;
    const int ln = 16 * (i / 4) + (mm % 16);
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < kSkWaves; ++w) sum += s_red[w][b][i % 4][ln];
    const int gcol = n0 + i;
    if (mm < m && gcol < n) y[(int64_t)mm * n + gcol] = sum + (bias ? bias[gcol] : 0.0f);
  }
}

// ---------------------------------------------------------------- tiled MFMA path

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kTiledThreads = 256;
constexpr int kLd = kBK + 8;  // padded LDS row stride (bf16 elements)

__global__ __launch_bounds__(kTiledThreads) void linear_tiled(
    const uint16_t* __restrict__ x, const uint32_t* __restrict__ packed,
    const uint32_t* __restrict__ sign, const float* __restrict__ scale,
    const float* __restrict__ bias, int m, int n, int k, Levels lv, float* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) uint16_t s_a[kBM * kLd];
  __shared__ __attribute__((aligned(16))) uint16_t s_b[kBN * kLd];
  __shared__ uint16_t s_lut[kBN * 16];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * kBM, n0 = blockIdx.x * kBN;
  const int kwords = k / 8, swords = k / 32;

  for (int i = tid; i < kBN * 16; i += kTiledThreads) {
    const int gn = n0 + (i >> 4);
    s_lut[i] = (uint16_t)lut_entry(lv, i & 15, gn < n ? scale[gn] : 0.0f);
  }

  floatx16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // weight staging: thread -> row tid/2, 32 k values (four packed words)
  const int br = tid >> 1, bh = tid & 1;
  const int bgn = n0 + br;

  for (int k0 = 0; k0 < k; k0 += kBK) {
    __syncthreads();  // previous tile consumed; tables ready on the first pass
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + kTiledThreads * i;
      const int r = c >> 3, cc = c & 7;
      const int gm = m0 + r, gk = k0 + cc * 8;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (gm < m && gk < k) v = *reinterpret_cast<const uint4*>(x + (int64_t)gm * k + gk);
      *reinterpret_cast<uint4*>(s_a + r * kLd + cc * 8) = v;
    }
    {
      const int gk = k0 + 32 * bh;
      uint4 pw = make_uint4(0u, 0u, 0u, 0u);
      uint32_t sw = 0u;
      if (bgn < n && gk < k) {
        pw = *reinterpret_cast<const uint4*>(packed + (int64_t)bgn * kwords + gk / 8);
        sw = sign[(int64_t)bgn * swords + gk / 32];
      }
      const uint16_t* lut = s_lut + br * 16;
      const uint32_t pws[4] = {pw.x, pw.y, pw.z, pw.w};
      uint32_t o[16];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          uint32_t h = lut[(pws[j] >> (4 * i)) & 15u];
          h |= ((sw >> (8 * j + i)) & 1u) << 15;
          if (i & 1) o[4 * j + (i >> 1)] |= h << 16;
          else o[4 * j + (i >> 1)] = h;
        }
      uint4* dst = reinterpret_cast<uint4*>(s_b + br * kLd + 32 * bh);
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[j] = make_uint4(o[4 * j], o[4 * j + 1], o[4 * j + 2], o[4 * j + 3]);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 16) {
      bf16x8_t a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8_t*>(s_a + (wm * 64 + i * 32 + (lane & 31)) * kLd + kk +
                                                  8 * (lane >> 5));
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = *reinterpret_cast<const bf16x8_t*>(s_b + (wn * 64 + j * 32 + (lane & 31)) * kLd + kk +
                                                  8 * (lane >> 5));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }

  // 32x32 accumulator layout: register e of lane l is row 8*(e/4) + 4*(l/32) + e%4,
  // column l%32.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + j * 32 + (lane & 31);
      const float bv = (bias && col < n) ? bias[col] : 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (row < m && col < n) y[(int64_t)row * n + col] = acc[i][j][e] + bv;
      }
    }
}

}  // namespace

size_t linear_workspace_bytes(int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_linear(const uint16_t* x, const uint32_t* packed, const uint32_t* sign,
                         const float* scale, const float* bias, int64_t m, int64_t n, int64_t k,
                         const Levels& lv, float* y, void*, hipStream_t stream) {
  if (m <= kSkinnyMaxM) {
    const int64_t blocks = (n + kSkRows - 1) / kSkRows;
    hipLaunchKernelGGL(linear_skinny, dim3((unsigned)blocks), dim3(kSkWaves * kWave), 0, stream, x,
                       packed, sign, scale, bias, (int)m, (int)n, (int)k, lv, y);
  } else {
    const dim3 grid((unsigned)((n + kBN - 1) / kBN), (unsigned)((m + kBM - 1) / kBM));
    hipLaunchKernelGGL(linear_tiled, grid, dim3(kTiledThreads), 0, stream, x, packed, sign, scale,
                       bias, (int)m, (int)n, (int)k, lv, y);
  }
  return hipGetLastError();
}

}  // namespace opq
