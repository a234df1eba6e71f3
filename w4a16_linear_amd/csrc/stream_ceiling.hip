// Streaming ceiling for the HBM-bound kernels (a measuring aid for the
// benchmark, not part of the OPQ interface; built as libopq_ceiling.so).
//
// quantize and dequantize read one row of k weights and write one row of codes
// (or the reverse); their floor on this GPU is what plain row streaming of the
// same bytes reaches.  This kernel reads `rd_bytes` and writes `wr_bytes` per
// row with 16-byte accesses and no arithmetic beyond an xor that keeps the
// reads live, one row per block at a time.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kThreads = 256;
constexpr int kMaxBlocks = 256 * 8;  // eight per CU on 256 CUs, each looping over rows

__global__ __launch_bounds__(kThreads) void stream_rows(const uint4* __restrict__ src,
                                                        uint4* __restrict__ dst, int64_t rows,
                                                        int rd, int wr) {
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const uint4* s = src + r * rd;
    uint4* d = dst + r * wr;
    uint32_t acc = 0u;
    for (int i = threadIdx.x; i < rd; i += kThreads) {
      const uint4 v = s[i];
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    for (int i = threadIdx.x; i < wr; i += kThreads)
      d[i] = make_uint4(acc, acc ^ (uint32_t)i, acc, (uint32_t)r);
  }
}

}  // namespace

// rows x rd_bytes read from src and rows x wr_bytes written to dst (device
// pointers, 16-byte aligned; byte counts multiples of 16, each below 2^31) on
// `stream`.  Returns 0, 1 for bad arguments, or 2 when the launch fails.
extern "C" int opq_ceiling_stream_rows(const void* src, void* dst, int64_t rows, int64_t rd_bytes,
                                       int64_t wr_bytes, void* stream) {
  if (rows < 0 || rd_bytes < 0 || wr_bytes < 0 || rd_bytes % 16 || wr_bytes % 16 ||
      rd_bytes >= (int64_t(1) << 31) || wr_bytes >= (int64_t(1) << 31) ||
      (rows && rd_bytes && !src) || (rows && wr_bytes && !dst) ||
      (reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16)
    return 1;
  if (rows == 0) return 0;
  const int64_t blocks = rows < kMaxBlocks ? rows : kMaxBlocks;
  hipLaunchKernelGGL(stream_rows, dim3((unsigned)blocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(src),
                     static_cast<uint4*>(dst), rows, (int)(rd_bytes / 16), (int)(wr_bytes / 16));
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
