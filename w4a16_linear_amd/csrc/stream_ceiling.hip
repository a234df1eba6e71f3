// Streaming ceiling for the HBM-bound kernels (a measuring aid for the
// benchmark, not part of the OPQ interface; built as libopq_ceiling.so).
//
// quantize and dequantize read one row of k weights and write one row of codes
// (or the reverse); their floor on this GPU is what plain streaming of the
// same bytes reaches.  This kernel moves exactly those bytes and does no
// arithmetic beyond an xor that keeps the reads live.  It is tuned for the
// memory system, not for the row structure: consecutive rows form tiles of
// about 16 KB on the longer side (read and written parts each contiguous, in
// the rows' own proportion), every thread keeps four 16-byte loads in flight,
// the stores are nontemporal, the loads too when a row reads more than it
// writes, and up to 8192 blocks loop over the tiles.  In a sweep over tile size
// (8-32 KB), loads in flight (4, 8), block count (2048, 8192) and cache hints
// this form was the fastest plain streaming kernel tried.  With inputs rotated
// past the 256 MB Infinity Cache it moves a 20480 x 3840 layer's bytes at 0.75
// of 8 TB/s in the quantize mix (3.2 : 1 read : write) and 0.73 in the
// dequantize mix (1 : 3.2); gigabyte streams reach 0.79-0.88 for reads alone and
// 0.65-0.69 for writes alone.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kThreads = 256;
constexpr int kInFlight = 4;        // 16-byte loads per thread per pass
constexpr int kTileUnits = 1024;    // 16-byte units on the longer side of a tile
constexpr int kMaxBlocks = 8192;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// rows x rd units read from src and rows x wr units written to dst (16-byte
// units), rpt rows per tile.
template <bool kNtLoad>
__global__ __launch_bounds__(kThreads) void stream_tiles(const uint4* __restrict__ src,
                                                         uint4* __restrict__ dst, int64_t rows,
                                                         int rd, int wr, int rpt) {
  const int64_t ntiles = (rows + rpt - 1) / rpt;
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t r0 = t * rpt;
    const int nr = (int)(rows - r0 < rpt ? rows - r0 : rpt);
    const int tr = nr * rd, tw = nr * wr;
    const uint4* s = src + r0 * rd;
    u32x4* d = reinterpret_cast<u32x4*>(dst + r0 * wr);
    uint32_t acc = 0u;
    for (int base = threadIdx.x; base < tr; base += kThreads * kInFlight) {
      uint4 v[kInFlight];
#pragma unroll
      for (int u = 0; u < kInFlight; ++u) {
        const int i = base + u * kThreads;
        if (i < tr) {
          if constexpr (kNtLoad) {
            const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(s + i));
            v[u] = make_uint4(x.x, x.y, x.z, x.w);
          } else {
            v[u] = s[i];
          }
        } else {
          v[u] = make_uint4(0u, 0u, 0u, 0u);
        }
      }
#pragma unroll
      for (int u = 0; u < kInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (int i = threadIdx.x; i < tw; i += kThreads) {
      const u32x4 o = {acc, (uint32_t)i, (uint32_t)t, 0u};
      __builtin_nontemporal_store(o, d + i);
    }
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
  if (rows == 0 || (rd_bytes == 0 && wr_bytes == 0)) return 0;
  const int rd = (int)(rd_bytes / 16), wr = (int)(wr_bytes / 16);
  const int longer = rd > wr ? rd : wr;
  // rows per tile: the tile's longer side stays near kTileUnits (and its unit
  // counts below 2^31: a row of more than kTileUnits units is a tile alone)
  const int rpt = longer >= kTileUnits ? 1 : kTileUnits / longer;
  const int64_t ntiles = (rows + rpt - 1) / rpt;
  const int64_t blocks = ntiles < kMaxBlocks ? ntiles : kMaxBlocks;
  hipLaunchKernelGGL(rd > wr ? stream_tiles<true> : stream_tiles<false>, dim3((unsigned)blocks),
                     dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(src),
                     static_cast<uint4*>(dst), rows, rd, wr, rpt);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
