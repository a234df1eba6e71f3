// Internal interface between the C ABI (opq_api.cpp), the host tables
// (tables.cpp) and the kernel launchers (*.hip).  Not installed.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace opq {

constexpr int kLevels = 15;  // 4-bit magnitude codes 0..15

// A launch's grid counts work-items in 32 bits; launchers whose grid grows with
// the rows split larger inputs into launches of at most this many.
constexpr int64_t kMaxLaunchThreads = int64_t(1) << 31;

// Decision points T_k (k = 1..15) of round(15 u^alpha), passed by value.
struct DecisionPoints {
  float t[kLevels];
};

// Reconstruction levels G_q = (q/15)^(1/alpha), q = 0..15, passed by value.
struct Levels {
  double g[kLevels + 1];
};

// tables.cpp (host only)
bool decision_points(float alpha, float out[kLevels]);
void levels(float alpha, double out[kLevels + 1]);

// Other code widths: b bits give L = 2^b - 1 levels (3 <= b <= 6).
constexpr int kMaxLevels = 63;
struct DecisionPointsN {
  float t[kMaxLevels];
  int n;  // L
};
struct LevelsN {
  double g[kMaxLevels + 1];
  int n;  // L
};
bool decision_points_n(float alpha, int L, float* out);  // out[L]
void levels_n(float alpha, int L, double* out);          // out[L + 1]

// quantize.hip
hipError_t launch_quantize(const void* w, bool w_is_bf16, int64_t n, int64_t k,
                           const DecisionPoints& dp, uint32_t* packed, uint32_t* sign,
                           float* scale, hipStream_t stream);

// quantize.hip: per-row (sum w^2, sum (w - w')^2) without storing the stored form
bool error_sums_supported(const DecisionPoints& dp, int64_t k);
hipError_t launch_error_sums(const void* w, bool w_is_bf16, int64_t n, int64_t k,
                             const DecisionPoints& dp, const Levels& lv, double* row_sums,
                             hipStream_t stream);

// dequantize.hip
hipError_t launch_dequantize(const uint32_t* packed, const uint32_t* sign, const float* scale,
                             int64_t n, int64_t k, const Levels& lv, uint16_t* out,
                             hipStream_t stream);

// linear.hip
size_t linear_workspace_bytes(int64_t m, int64_t n, int64_t k);
hipError_t launch_linear(const uint16_t* x, const uint32_t* packed, const uint32_t* sign,
                         const float* scale, const float* bias, int64_t m, int64_t n, int64_t k,
                         const Levels& lv, void* y, bool y_bf16, void* workspace,
                         hipStream_t stream);

// linear.hip: a fixed device array per GPU (the allocation-free b-bit linear
// layer) and its address on the current device (nullptr if the runtime
// cannot report it)
constexpr size_t kNoAllocScratchBytes = size_t(160) << 20;
void* noalloc_scratch();

// linear.hip: y = x W'^T (+ bias) with W' bfloat16 [n][k] in device memory
hipError_t launch_linear_dense(const uint16_t* x, const uint16_t* wd, const float* bias, int64_t m,
                               int64_t n, int64_t k, void* y, bool y_bf16, hipStream_t stream);

// b-bit codes (3..6), codes of a row as a little-endian bit stream along k.
// quantize.hip
bool bits_supported(const DecisionPointsN& dp, int64_t k);
hipError_t launch_quantize_bits(const void* w, bool w_is_bf16, int64_t n, int64_t k, int bits,
                                const DecisionPointsN& dp, const LevelsN& lv, uint32_t* packed,
                                uint32_t* sign, float* scale, double* row_sums,
                                hipStream_t stream);
// dequantize.hip
hipError_t launch_dequantize_bits(const uint32_t* packed, const uint32_t* sign,
                                  const float* scale, int64_t n, int64_t k, int bits,
                                  const LevelsN& lv, uint16_t* out, bool stream_out,
                                  hipStream_t stream);  // stream_out: nontemporal stores

// Group-wise form (one float16 max per `gs` weights along k).
// quantize.hip: alpha has a bucket grid and G_1 * 2^-24 is a normal binary32
bool grouped_supported(const DecisionPoints& dp, const Levels& lv);
hipError_t launch_quantize_grouped(const void* w, bool w_is_bf16, int64_t n, int64_t k, int gs,
                                   const DecisionPoints& dp, uint32_t* packed, uint32_t* sign,
                                   uint16_t* scale16, hipStream_t stream);
// dequantize.hip
hipError_t launch_dequantize_grouped(const uint32_t* packed, const uint32_t* sign,
                                     const uint16_t* scale16, int64_t n, int64_t k, int gs,
                                     const Levels& lv, uint16_t* out, hipStream_t stream);
// linear.hip
hipError_t launch_linear_grouped(const uint16_t* x, const uint32_t* packed, const uint32_t* sign,
                                 const uint16_t* scale16, const float* bias, int64_t m, int64_t n,
                                 int64_t k, int gs, const Levels& lv, void* y, bool y_bf16,
                                 void* workspace, hipStream_t stream);

}  // namespace opq
