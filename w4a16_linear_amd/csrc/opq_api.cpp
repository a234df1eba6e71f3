// The C ABI of libopq (include/opq.h): argument checks in the documented
// order, host tables, then one launch on the caller's stream.
#include "opq.h"

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>

#include "opq_internal.hpp"

namespace {

constexpr int64_t kMaxK = 65536;
// the skinny linear kernel takes a block of 512 threads per 16 weight rows
constexpr int64_t kMaxLinearN = int64_t(1) << 26;

// NULL (allowed for an empty array) counts as aligned.
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool alpha_ok(float a) { return std::isfinite(a) && a > 0.0f; }

bool shape_ok(int64_t n, int64_t k) { return n >= 0 && k >= 0 && k % 32 == 0; }

bool bits_ok(int bits) { return bits >= 3 && bits <= 6; }

// Decision points and levels of b-bit codes (2^b - 1 levels).
bool bits_tables(float alpha, int bits, opq::DecisionPointsN& dp, opq::LevelsN& lv) {
  const int L = (1 << bits) - 1;
  dp.n = lv.n = L;
  for (int i = L; i < opq::kMaxLevels; ++i) dp.t[i] = 2.0f;
  for (int i = L + 1; i <= opq::kMaxLevels; ++i) lv.g[i] = 0.0;
  if (!opq::decision_points_n(alpha, L, dp.t)) return false;
  opq::levels_n(alpha, L, lv.g);
  return true;
}

bool group_ok(int64_t k, int64_t gs) {
  return (gs == 32 || gs == 64 || gs == 128 || gs == 256) && k % gs == 0;
}

int hip_status(hipError_t e) { return e == hipSuccess ? OPQ_OK : OPQ_ERR_HIP; }

}  // namespace

extern "C" {

int opq_abi_version(void) { return OPQ_ABI_VERSION; }

const char* opq_status_str(int status) {
  switch (status) {
    case OPQ_OK: return "ok";
    case OPQ_ERR_NULL: return "a required pointer is NULL";
    case OPQ_ERR_SHAPE:
      return "bad shape: sizes must be >= 0, k a multiple of 32 (and of the group, which is "
             "32, 64, 128 or 256); bits 3, 4, 5 or 6";
    case OPQ_ERR_ALPHA: return "alpha must be finite and > 0";
    case OPQ_ERR_ALIGN: return "every array must be 16-byte aligned";
    case OPQ_ERR_DTYPE: return "unknown dtype code";
    case OPQ_ERR_WORKSPACE: return "workspace smaller than opq_linear_workspace_bytes()";
    case OPQ_ERR_UNSUPPORTED: return "size beyond what the kernels handle";
    case OPQ_ERR_HIP: return "the HIP runtime refused a launch";
    default: return "unknown status";
  }
}

int opq_decision_points(float alpha, float* out_t) {
  if (!out_t) return OPQ_ERR_NULL;
  if (!alpha_ok(alpha)) return OPQ_ERR_ALPHA;
  return opq::decision_points(alpha, out_t) ? OPQ_OK : OPQ_ERR_ALPHA;
}

int opq_levels(float alpha, double* out_g) {
  if (!out_g) return OPQ_ERR_NULL;
  if (!alpha_ok(alpha)) return OPQ_ERR_ALPHA;
  opq::levels(alpha, out_g);
  return OPQ_OK;
}

int opq_quantize(const void* w, int w_dtype, int64_t n, int64_t k, float alpha,
                 uint32_t* packed, uint32_t* sign, float* scale, void* stream) {
  const bool nk = n > 0 && k > 0;
  if ((nk && (!w || !packed || !sign)) || (n > 0 && !scale)) return OPQ_ERR_NULL;
  if (!shape_ok(n, k)) return OPQ_ERR_SHAPE;
  if (!alpha_ok(alpha)) return OPQ_ERR_ALPHA;
  if (!aligned16(w) || !aligned16(packed) || !aligned16(sign) || !aligned16(scale))
    return OPQ_ERR_ALIGN;
  if (w_dtype != OPQ_F32 && w_dtype != OPQ_BF16) return OPQ_ERR_DTYPE;
  if (k > kMaxK) return OPQ_ERR_UNSUPPORTED;
  if (n == 0) return OPQ_OK;
  opq::DecisionPoints dp;
  if (!opq::decision_points(alpha, dp.t)) return OPQ_ERR_ALPHA;
  return hip_status(opq::launch_quantize(w, w_dtype == OPQ_BF16, n, k, dp, packed, sign, scale,
                                         static_cast<hipStream_t>(stream)));
}

int opq_error_sums(const void* w, int w_dtype, int64_t n, int64_t k, float alpha,
                   double* row_sums, void* stream) {
  if ((n > 0 && k > 0 && !w) || (n > 0 && !row_sums)) return OPQ_ERR_NULL;
  if (!shape_ok(n, k)) return OPQ_ERR_SHAPE;
  if (!alpha_ok(alpha)) return OPQ_ERR_ALPHA;
  if (!aligned16(w) || !aligned16(row_sums)) return OPQ_ERR_ALIGN;
  if (w_dtype != OPQ_F32 && w_dtype != OPQ_BF16) return OPQ_ERR_DTYPE;
  if (n == 0) return OPQ_OK;
  opq::DecisionPoints dp;
  if (!opq::decision_points(alpha, dp.t)) return OPQ_ERR_ALPHA;
  if (!opq::error_sums_supported(dp, k)) return OPQ_ERR_UNSUPPORTED;
  opq::Levels lv;  // k == 0 runs the kernel too: it writes zero sums
  opq::levels(alpha, lv.g);
  return hip_status(opq::launch_error_sums(w, w_dtype == OPQ_BF16, n, k, dp, lv, row_sums,
                                           static_cast<hipStream_t>(stream)));
}

int opq_dequantize(const uint32_t* packed, const uint32_t* sign, const float* scale, int64_t n,
                   int64_t k, float alpha, uint16_t* w_out, void* stream) {
  if (n > 0 && k > 0 && (!packed || !sign || !scale || !w_out)) return OPQ_ERR_NULL;
  if (!shape_ok(n, k)) return OPQ_ERR_SHAPE;
  if (!alpha_ok(alpha)) return OPQ_ERR_ALPHA;
  if (!aligned16(packed) || !aligned16(sign) || !aligned16(scale) || !aligned16(w_out))
    return OPQ_ERR_ALIGN;
  if (n == 0 || k == 0) return OPQ_OK;
  if (k > kMaxK) return OPQ_ERR_UNSUPPORTED;
  opq::Levels lv;
  opq::levels(alpha, lv.g);
  return hip_status(opq::launch_dequantize(packed, sign, scale, n, k, lv, w_out,
                                           static_cast<hipStream_t>(stream)));
}

size_t opq_linear_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  if (m < 0 || !shape_ok(n, k) || k > kMaxK || n > kMaxLinearN) return 0;
  return opq::linear_workspace_bytes(m, n, k);
}

int opq_linear(const uint16_t* x, const uint32_t* packed, const uint32_t* sign, const float* scale,
               const float* bias, int64_t m, int64_t n, int64_t k, float alpha, void* y,
               int y_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if ((m > 0 && k > 0 && !x) || (n > 0 && k > 0 && (!packed || !sign)) || (n > 0 && !scale) ||
      (m > 0 && n > 0 && !y))
    return OPQ_ERR_NULL;
  if (m < 0 || !shape_ok(n, k)) return OPQ_ERR_SHAPE;
  if (!alpha_ok(alpha)) return OPQ_ERR_ALPHA;
  if (!aligned16(x) || !aligned16(packed) || !aligned16(sign) || !aligned16(scale) ||
      !aligned16(y) || (bias && !aligned16(bias)) || (workspace && !aligned16(workspace)))
    return OPQ_ERR_ALIGN;
  if (y_dtype != OPQ_F32 && y_dtype != OPQ_BF16) return OPQ_ERR_DTYPE;
  const size_t need = opq_linear_workspace_bytes(m, n, k);
  if (workspace_bytes < need || (need > 0 && !workspace)) return OPQ_ERR_WORKSPACE;
  if (m == 0 || n == 0) return OPQ_OK;
  if (k > kMaxK || n > kMaxLinearN) return OPQ_ERR_UNSUPPORTED;
  opq::Levels lv;
  opq::levels(alpha, lv.g);
  return hip_status(opq::launch_linear(x, packed, sign, scale, bias, m, n, k, lv, y,
                                       y_dtype == OPQ_BF16, workspace,
                                       static_cast<hipStream_t>(stream)));
}

int opq_quantize_bits(const void* w, int w_dtype, int64_t n, int64_t k, int bits, float alpha,
                      uint32_t* packed, uint32_t* sign, float* scale, void* stream) {
  if (bits == 4) return opq_quantize(w, w_dtype, n, k, alpha, packed, sign, scale, stream);
  const bool nk = n > 0 && k > 0;
  if ((nk && (!w || !packed || !sign)) || (n > 0 && !scale)) return OPQ_ERR_NULL;
  if (!shape_ok(n, k) || !bits_ok(bits)) return OPQ_ERR_SHAPE;
  if (!alpha_ok(alpha)) return OPQ_ERR_ALPHA;
  if (!aligned16(w) || !aligned16(packed) || !aligned16(sign) || !aligned16(scale))
    return OPQ_ERR_ALIGN;
  if (w_dtype != OPQ_F32 && w_dtype != OPQ_BF16) return OPQ_ERR_DTYPE;
  if (n == 0) return OPQ_OK;
  opq::DecisionPointsN dp;
  opq::LevelsN lv;
  if (!bits_tables(alpha, bits, dp, lv)) return OPQ_ERR_ALPHA;
  if (!opq::bits_supported(dp, k)) return OPQ_ERR_UNSUPPORTED;
  return hip_status(opq::launch_quantize_bits(w, w_dtype == OPQ_BF16, n, k, bits, dp, lv, packed,
                                              sign, scale, nullptr,
                                              static_cast<hipStream_t>(stream)));
}

int opq_dequantize_bits(const uint32_t* packed, const uint32_t* sign, const float* scale,
                        int64_t n, int64_t k, int bits, float alpha, uint16_t* w_out,
                        void* stream) {
  if (bits == 4) return opq_dequantize(packed, sign, scale, n, k, alpha, w_out, stream);
  if (n > 0 && k > 0 && (!packed || !sign || !scale || !w_out)) return OPQ_ERR_NULL;
  if (!shape_ok(n, k) || !bits_ok(bits)) return OPQ_ERR_SHAPE;
  if (!alpha_ok(alpha)) return OPQ_ERR_ALPHA;
  if (!aligned16(packed) || !aligned16(sign) || !aligned16(scale) || !aligned16(w_out))
    return OPQ_ERR_ALIGN;
  if (n == 0 || k == 0) return OPQ_OK;
  if (k > kMaxK) return OPQ_ERR_UNSUPPORTED;
  opq::DecisionPointsN dp;
  opq::LevelsN lv;
  if (!bits_tables(alpha, bits, dp, lv)) return OPQ_ERR_ALPHA;
  return hip_status(opq::launch_dequantize_bits(packed, sign, scale, n, k, bits, lv, w_out, true,
                                                static_cast<hipStream_t>(stream)));
}

int opq_error_sums_bits(const void* w, int w_dtype, int64_t n, int64_t k, int bits, float alpha,
                        double* row_sums, void* stream) {
  if (bits == 4) return opq_error_sums(w, w_dtype, n, k, alpha, row_sums, stream);
  if ((n > 0 && k > 0 && !w) || (n > 0 && !row_sums)) return OPQ_ERR_NULL;
  if (!shape_ok(n, k) || !bits_ok(bits)) return OPQ_ERR_SHAPE;
  if (!alpha_ok(alpha)) return OPQ_ERR_ALPHA;
  if (!aligned16(w) || !aligned16(row_sums)) return OPQ_ERR_ALIGN;
  if (w_dtype != OPQ_F32 && w_dtype != OPQ_BF16) return OPQ_ERR_DTYPE;
  if (n == 0) return OPQ_OK;
  opq::DecisionPointsN dp;
  opq::LevelsN lv;
  if (!bits_tables(alpha, bits, dp, lv)) return OPQ_ERR_ALPHA;
  if (!opq::bits_supported(dp, k)) return OPQ_ERR_UNSUPPORTED;
  return hip_status(opq::launch_quantize_bits(w, w_dtype == OPQ_BF16, n, k, bits, dp, lv, nullptr,
                                              nullptr, nullptr, row_sums,
                                              static_cast<hipStream_t>(stream)));
}

int opq_quantize_grouped(const void* w, int w_dtype, int64_t n, int64_t k, int64_t group,
                         float alpha, uint32_t* packed, uint32_t* sign, uint16_t* scale16,
                         void* stream) {
  const bool nk = n > 0 && k > 0;
  if (nk && (!w || !packed || !sign || !scale16)) return OPQ_ERR_NULL;
  if (!shape_ok(n, k) || !group_ok(k, group)) return OPQ_ERR_SHAPE;
  if (!alpha_ok(alpha)) return OPQ_ERR_ALPHA;
  if (!aligned16(w) || !aligned16(packed) || !aligned16(sign) || !aligned16(scale16))
    return OPQ_ERR_ALIGN;
  if (w_dtype != OPQ_F32 && w_dtype != OPQ_BF16) return OPQ_ERR_DTYPE;
  if (!nk) return OPQ_OK;
  opq::DecisionPoints dp;
  if (!opq::decision_points(alpha, dp.t)) return OPQ_ERR_ALPHA;
  opq::Levels lv;
  opq::levels(alpha, lv.g);
  if (!opq::grouped_supported(dp, lv)) return OPQ_ERR_UNSUPPORTED;
  return hip_status(opq::launch_quantize_grouped(w, w_dtype == OPQ_BF16, n, k, (int)group, dp,
                                                 packed, sign, scale16,
                                                 static_cast<hipStream_t>(stream)));
}

int opq_dequantize_grouped(const uint32_t* packed, const uint32_t* sign, const uint16_t* scale16,
                           int64_t n, int64_t k, int64_t group, float alpha, uint16_t* w_out,
                           void* stream) {
  if (n > 0 && k > 0 && (!packed || !sign || !scale16 || !w_out)) return OPQ_ERR_NULL;
  if (!shape_ok(n, k) || !group_ok(k, group)) return OPQ_ERR_SHAPE;
  if (!alpha_ok(alpha)) return OPQ_ERR_ALPHA;
  if (!aligned16(packed) || !aligned16(sign) || !aligned16(scale16) || !aligned16(w_out))
    return OPQ_ERR_ALIGN;
  if (n == 0 || k == 0) return OPQ_OK;
  opq::DecisionPoints dp;
  if (!opq::decision_points(alpha, dp.t)) return OPQ_ERR_ALPHA;
  opq::Levels lv;
  opq::levels(alpha, lv.g);
  if (!opq::grouped_supported(dp, lv)) return OPQ_ERR_UNSUPPORTED;
  return hip_status(opq::launch_dequantize_grouped(packed, sign, scale16, n, k, (int)group, lv,
                                                   w_out, static_cast<hipStream_t>(stream)));
}

size_t opq_linear_bits_workspace_bytes(int64_t m, int64_t n, int64_t k, int bits) {
  if (bits == 4) return opq_linear_workspace_bytes(m, n, k);
  if (m <= 0 || n <= 0 || k <= 0 || !bits_ok(bits)) return 0;
  return ((size_t)n * (size_t)k * 2u + 255u) & ~(size_t)255u;  // W' as bfloat16
}

int opq_linear_bits(const uint16_t* x, const uint32_t* packed, const uint32_t* sign,
                    const float* scale, const float* bias, int64_t m, int64_t n, int64_t k, int bits,
                    float alpha, void* y, int y_dtype, void* workspace, size_t workspace_bytes,
                    void* stream) {
  if (bits == 4)
    return opq_linear(x, packed, sign, scale, bias, m, n, k, alpha, y, y_dtype, workspace,
                      workspace_bytes, stream);
  if ((m > 0 && k > 0 && !x) || (n > 0 && k > 0 && (!packed || !sign)) || (n > 0 && !scale) ||
      (m > 0 && n > 0 && !y))
    return OPQ_ERR_NULL;
  if (m < 0 || !shape_ok(n, k) || !bits_ok(bits)) return OPQ_ERR_SHAPE;
  if (!alpha_ok(alpha)) return OPQ_ERR_ALPHA;
  if (!aligned16(x) || !aligned16(packed) || !aligned16(sign) || !aligned16(scale) ||
      !aligned16(y) || (bias && !aligned16(bias)) || (workspace && !aligned16(workspace)))
    return OPQ_ERR_ALIGN;
  if (y_dtype != OPQ_F32 && y_dtype != OPQ_BF16) return OPQ_ERR_DTYPE;
  const size_t need = opq_linear_bits_workspace_bytes(m, n, k, bits);
  if (workspace_bytes < need || (need > 0 && !workspace)) return OPQ_ERR_WORKSPACE;
  if (m == 0 || n == 0) return OPQ_OK;
  if (k > kMaxK || n > kMaxLinearN) return OPQ_ERR_UNSUPPORTED;
  opq::DecisionPointsN dp;
  opq::LevelsN lv;
  if (!bits_tables(alpha, bits, dp, lv)) return OPQ_ERR_ALPHA;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  uint16_t* wd = static_cast<uint16_t*>(workspace);
  if (k > 0) {
    // W' stays in cache for the dense product that reads it next
    const int e =
        hip_status(opq::launch_dequantize_bits(packed, sign, scale, n, k, bits, lv, wd, false, st));
    if (e != OPQ_OK) return e;
  }
  return hip_status(opq::launch_linear_dense(x, wd, bias, m, n, k, y, y_dtype == OPQ_BF16, st));
}

int opq_linear_bits_noalloc(const uint16_t* x, const uint32_t* packed, const uint32_t* sign,
                            const float* scale, const float* bias, int64_t m, int64_t n, int64_t k,
                            int bits, float alpha, void* y, int y_dtype, void* stream) {
  const size_t need = opq_linear_bits_workspace_bytes(m, n, k, bits);  // 0 for invalid shapes
  if (need == 0)  // nothing to hold; argument errors come back from the call itself
    return opq_linear_bits(x, packed, sign, scale, bias, m, n, k, bits, alpha, y, y_dtype, nullptr,
                           0, stream);
  // Arguments first, as opq_linear_bits checks them: with no workspace and
  // need > 0 that call never launches, and answers OPQ_ERR_WORKSPACE once all
  // else is valid.
  const int st = opq_linear_bits(x, packed, sign, scale, bias, m, n, k, bits, alpha, y, y_dtype,
                                 nullptr, SIZE_MAX, nullptr);
  if (st != OPQ_ERR_WORKSPACE) return st;
  if (need > opq::kNoAllocScratchBytes) return OPQ_ERR_UNSUPPORTED;
  void* ws = opq::noalloc_scratch();
  if (!ws) return OPQ_ERR_HIP;
  return opq_linear_bits(x, packed, sign, scale, bias, m, n, k, bits, alpha, y, y_dtype, ws, need,
                         stream);
}

int opq_linear_grouped(const uint16_t* x, const uint32_t* packed, const uint32_t* sign,
                       const uint16_t* scale16, const float* bias, int64_t m, int64_t n,
                       int64_t k, int64_t group, float alpha, void* y, int y_dtype,
                       void* workspace, size_t workspace_bytes, void* stream) {
  if ((m > 0 && k > 0 && !x) || (n > 0 && k > 0 && (!packed || !sign || !scale16)) ||
      (m > 0 && n > 0 && !y))
    return OPQ_ERR_NULL;
  if (m < 0 || !shape_ok(n, k) || !group_ok(k, group)) return OPQ_ERR_SHAPE;
  if (!alpha_ok(alpha)) return OPQ_ERR_ALPHA;
  if (!aligned16(x) || !aligned16(packed) || !aligned16(sign) || !aligned16(scale16) ||
      !aligned16(y) || (bias && !aligned16(bias)) || (workspace && !aligned16(workspace)))
    return OPQ_ERR_ALIGN;
  if (y_dtype != OPQ_F32 && y_dtype != OPQ_BF16) return OPQ_ERR_DTYPE;
  if (m == 0 || n == 0) return OPQ_OK;  // the group-wise kernels use no workspace
  if (k > kMaxK || n > kMaxLinearN) return OPQ_ERR_UNSUPPORTED;
  opq::DecisionPoints dp;
  if (!opq::decision_points(alpha, dp.t)) return OPQ_ERR_ALPHA;
  opq::Levels lv;
  opq::levels(alpha, lv.g);
  if (!opq::grouped_supported(dp, lv)) return OPQ_ERR_UNSUPPORTED;
  return hip_status(opq::launch_linear_grouped(x, packed, sign, scale16, bias, m, n, k,
                                               (int)group, lv, y, y_dtype == OPQ_BF16, workspace,
                                               static_cast<hipStream_t>(stream)));
}

}  // extern "C"
