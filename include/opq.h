/*
 * libopq: OPQ (Optimal Power Quantization) 4-bit weights for AMD MI355X (gfx950).
 *
 * The method is the one on the model card "OPQ INT4 Z-Image"
 * (huggingpeers.co/models/dfytensor/OPQ-INT4-Z-Image):
 *   section "OPQ 原理"            u = |w| / max|w|,  v = u^alpha,  q = round(15 v),
 *                                  w' = sign(w) (q/15)^(1/alpha) max|w|;
 *   section "技术细节 / 存储格式"  4-bit magnitudes eight per uint32, a 1-bit sign
 *                                  plane thirty-two per uint32, one max per group;
 *   section "技术细节 / 推理解码"  decode q/15 -> ^(1/alpha) -> x sign x max;
 *   file list "opq_quantize.py (OPQLinear + replace_with_opq)": a linear layer
 *                                  that runs on the stored form.
 *
 * Format of the main calls (the card leaves these open; the group-wise and
 * other-width calls further down change only what they say they change):
 *   - one max per output row n, stored as float32 scale[n];
 *   - packed[n][k/8] (uint32): code of (n, k) in bits 4*(k%8) .. 4*(k%8)+3;
 *   - sign[n][k/32]  (uint32): bit k%32 is 1 exactly when w[n][k] < 0;
 *   - codes are exact: q = the integer nearest to 15 * u^alpha with
 *     u = |w| / max|w| the IEEE binary32 quotient (round to nearest even,
 *     subnormals kept); an exact half (only alpha = 1, u = 1/2) rounds up;
 *   - a row whose max is 0 gets scale 0, codes 0 and signs 0;
 *   - bfloat16 values travel as uint16 bit patterns;
 *   - the magnitude is 4 bits and the sign a separate bit, so a weight takes
 *     one of 31 values although the card calls the format "INT4".
 *
 * Conventions for every call:
 *   - matrices are row-major and dense (row stride = number of columns);
 *   - device pointers are memory of the current HIP device; host pointers are
 *     marked as such;
 *   - the caller owns every buffer (scratch comes in as a workspace argument);
 *     no call allocates, frees or synchronises; the library's only global
 *     state is a mutex-guarded memo of the per-alpha host tables, per kernel
 *     a once-computed occupancy figure, and the fixed device array of
 *     opq_linear_bits_noalloc (its address looked up once per device), so
 *     calls are reentrant and thread-safe; outputs must not overlap inputs;
 *   - `stream` is a hipStream_t (NULL = the default stream); work is enqueued
 *     on it and the call returns at once; faults inside kernels show up at the
 *     caller's next synchronisation;
 *   - a pointer may be NULL exactly when the array it points to has no
 *     elements (for example packed and sign when k == 0);
 *   - arguments are checked before anything is enqueued, in this order:
 *     null pointers (OPQ_ERR_NULL), shapes (OPQ_ERR_SHAPE), alpha
 *     (OPQ_ERR_ALPHA), 16-byte alignment of every array (OPQ_ERR_ALIGN),
 *     dtype codes (OPQ_ERR_DTYPE), workspace size (OPQ_ERR_WORKSPACE);
 *     with an error nothing is enqueued;
 *   - n == 0 or m == 0 is a valid empty call (OPQ_OK, nothing enqueued);
 *   - k must be a multiple of 32 (one sign word); n, m are free;
 *   - alpha must be finite and > 0, and every call on one set of weights must
 *     get the same binary32 alpha (the stored form does not record it);
 *   - weights must be finite; with NaN or Inf the codes are unspecified.
 */
#ifndef OPQ_H
#define OPQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OPQ_ABI_VERSION 6

typedef enum {
  OPQ_OK = 0,
  OPQ_ERR_NULL = 1,        /* a required pointer is NULL */
  OPQ_ERR_SHAPE = 2,       /* negative size, or k not a multiple of 32 */
  OPQ_ERR_ALPHA = 3,       /* alpha not finite or not > 0 */
  OPQ_ERR_ALIGN = 4,       /* an array is not 16-byte aligned */
  OPQ_ERR_DTYPE = 5,       /* unknown dtype code */
  OPQ_ERR_WORKSPACE = 6,   /* workspace smaller than opq_linear_workspace_bytes() */
  OPQ_ERR_UNSUPPORTED = 7, /* a size beyond what the kernels handle */
  OPQ_ERR_HIP = 8          /* the HIP runtime refused a launch */
} opq_status;

typedef enum { OPQ_F32 = 0, OPQ_BF16 = 1 } opq_dtype;

/* ABI version of the loaded library (OPQ_ABI_VERSION). */
int opq_abi_version(void);

/* Static text for a status code; never NULL. */
const char* opq_status_str(int status);

/*
 * Decision points of the quantizer ("OPQ 原理": q = round(15 u^alpha)).
 * Host only, no GPU needed.  out_t (host, 15 floats) receives T_k, k = 1..15:
 * the smallest binary32 t with 15 t^alpha >= k - 1/2.  For binary32 u in
 * [0, 1] the code is the number of k with u >= T_k.  These are the values the
 * quantize kernel compares against.
 * Errors: OPQ_ERR_NULL, OPQ_ERR_ALPHA.
 */
int opq_decision_points(float alpha, float* out_t);

/*
 * Reconstruction levels ("推理解码": (q/15)^(1/alpha)).  Host only.
 * out_g (host, 16 doubles) receives G_q = (q/15)^(1/alpha) in double, q = 0..15;
 * G_0 = 0 and G_15 = 1 exactly.  A row with scale m reconstructs code q as the
 * bfloat16 nearest to G_q * m (one rounding); dequantize and linear both use it.
 * Errors: OPQ_ERR_NULL, OPQ_ERR_ALPHA.
 */
int opq_levels(float alpha, double* out_g);

/*
 * Quantize ("OPQ 原理", "存储格式").
 *   w       device, [n][k] of float32 (w_dtype OPQ_F32) or bfloat16 (OPQ_BF16)
 *   packed  device out, [n][k/8] uint32 magnitudes
 *   sign    device out, [n][k/32] uint32 sign plane
 *   scale   device out, [n] float32 = max_k |w[n][k]| (exact)
 * k <= 65536.  Errors: OPQ_ERR_NULL, OPQ_ERR_SHAPE, OPQ_ERR_ALPHA,
 * OPQ_ERR_ALIGN, OPQ_ERR_DTYPE, OPQ_ERR_UNSUPPORTED, OPQ_ERR_HIP.
 */
int opq_quantize(const void* w, int w_dtype, int64_t n, int64_t k, float alpha,
                 uint32_t* packed, uint32_t* sign, float* scale, void* stream);

/*
 * Reconstruction error for choosing alpha ("OPQ 原理": OPQ against uniform
 * rounding, which alpha = 1 is; "为什么 α=0.73？": alpha sits in the flat optimum
 * of this error).  Quantizes w as opq_quantize would, reconstructs it as
 * opq_dequantize would, and stores nothing but, per row,
 *   row_sums[2i]     = sum_k w[i][k]^2
 *   row_sums[2i + 1] = sum_k (w[i][k] - w'[i][k])^2
 * (binary32 over each wave's at most 4096 elements, then double across waves
 * in a fixed order: reproducible, and within 70 * 2^-24 relative of the exact
 * sums of these nonnegative terms).  SNR in dB
 * over a tensor is 10 log10(sum of the first column / sum of the second).
 *   w         device, [n][k] float32 (OPQ_F32) or bfloat16 (OPQ_BF16)
 *   row_sums  device out, [n][2] double
 * k <= 16384, and alpha must have a separating bucket grid (every alpha in
 * [0.05, 60] does); otherwise OPQ_ERR_UNSUPPORTED.
 * Errors: OPQ_ERR_NULL, OPQ_ERR_SHAPE, OPQ_ERR_ALPHA, OPQ_ERR_ALIGN,
 * OPQ_ERR_DTYPE, OPQ_ERR_UNSUPPORTED, OPQ_ERR_HIP.
 */
int opq_error_sums(const void* w, int w_dtype, int64_t n, int64_t k, float alpha,
                   double* row_sums, void* stream);

/*
 * Dequantize ("推理解码").
 *   packed, sign, scale  device, as written by opq_quantize
 *   w_out   device out, [n][k] bfloat16: bf16(G_q * scale[n]) with the sign
 *           applied; code 0 gives +0.0
 * k <= 65536.  Errors: OPQ_ERR_NULL, OPQ_ERR_SHAPE, OPQ_ERR_ALPHA, OPQ_ERR_ALIGN,
 * OPQ_ERR_UNSUPPORTED, OPQ_ERR_HIP.
 */
int opq_dequantize(const uint32_t* packed, const uint32_t* sign, const float* scale,
                   int64_t n, int64_t k, float alpha, uint16_t* w_out, void* stream);

/*
 * Bytes of device workspace opq_linear needs for this shape (0 means none;
 * the workspace pointer may then be NULL).  Nonzero only where the tiled
 * layer splits k: m > 128 with k a multiple of 64, whose 256 x 256 output
 * tiles would cover at most a quarter of the 256 CUs (for example m = 1024,
 * n = 3840), and which the call does not run as 64-row slices of x.  It then keeps S
 * float32 partial sums per output: S * m * n * 4 bytes rounded up to 256, at
 * most 128 MiB, S chosen from the shape alone.  0 for every other shape.
 */
size_t opq_linear_workspace_bytes(int64_t m, int64_t n, int64_t k);

/*
 * W4A16 linear layer on the stored form (the card's OPQLinear):
 *   y[m][n] = sum_k x[m][k] * W'[n][k] (+ bias[n])
 * with W'[n][k] = the bfloat16 reconstruction that opq_dequantize writes,
 * made on chip, and float32 accumulation.
 *   x       device, [m][k] bfloat16 activations
 *   packed, sign, scale  device, as written by opq_quantize for W[n][k]
 *   bias    device, [n] float32, or NULL for none
 *   y       device out, [m][n] of float32 (y_dtype OPQ_F32) or bfloat16
 *           (OPQ_BF16: the float32 result rounded to nearest even)
 *   workspace, workspace_bytes  device scratch of at least
 *           opq_linear_workspace_bytes(m, n, k) bytes (NULL when that is 0):
 *           the split-k partial sums, added in slice order by a second kernel
 *           on the same stream.  It needs no initialisation and is
 *           overwritten, so one buffer serves any number of calls (of any
 *           shape) in one stream; calls that may run at the same time (other
 *           streams) need buffers of their own.
 * The sum order is fixed for a given shape, so results are reproducible bit
 * for bit.  k <= 65536 and n <= 2^26 (OPQ_ERR_UNSUPPORTED otherwise).
 * Errors: OPQ_ERR_NULL, OPQ_ERR_SHAPE, OPQ_ERR_ALPHA, OPQ_ERR_ALIGN,
 * OPQ_ERR_DTYPE, OPQ_ERR_WORKSPACE, OPQ_ERR_UNSUPPORTED, OPQ_ERR_HIP.
 */
int opq_linear(const uint16_t* x, const uint32_t* packed, const uint32_t* sign,
               const float* scale, const float* bias, int64_t m, int64_t n, int64_t k,
               float alpha, void* y, int y_dtype, void* workspace, size_t workspace_bytes,
               void* stream);

/*
 * Other code widths.  The configuration section of the card offers 3, 4, 5 or
 * 6 bits ("OPQ_BITS"); its formulas are written for 4 (x 15).  Here b bits
 * use 2^b - 1 in place of 15 everywhere: q = the integer nearest to
 * (2^b - 1) u^alpha (halves up), reconstruction bf16(G_q m) with
 * G_q = (q / (2^b - 1))^(1/alpha).  The sign plane and the per-row float32
 * scale are as for 4 bits.  The card gives no packing for b != 4; here the
 * codes of a row form a little-endian bit stream along k: code k occupies bits
 * b*k .. b*k + b - 1 of the row, so 32 codes fill b uint32 words and packed is
 * [n][k*b/32].  For b = 4 this is exactly the layout of opq_quantize, and
 * these calls give the same results as the 4-bit ones.
 *   bits     3, 4, 5 or 6 (OPQ_ERR_SHAPE otherwise)
 * The 4-bit linear layer (opq_linear) decodes on chip; opq_linear_bits below
 * serves the other widths.
 */

/*
 * Quantize with b-bit codes: w device [n][k] float32 or bfloat16; packed
 * [n][k*bits/32], sign [n][k/32], scale [n] device outputs.  For bits != 4,
 * k <= 16384 and alpha must have a separating bucket grid (every alpha in
 * [0.1, 10] has one for 6 bits); otherwise OPQ_ERR_UNSUPPORTED.  Errors:
 * OPQ_ERR_NULL, OPQ_ERR_SHAPE, OPQ_ERR_ALPHA, OPQ_ERR_ALIGN, OPQ_ERR_DTYPE,
 * OPQ_ERR_UNSUPPORTED, OPQ_ERR_HIP.
 */
int opq_quantize_bits(const void* w, int w_dtype, int64_t n, int64_t k, int bits, float alpha,
                      uint32_t* packed, uint32_t* sign, float* scale, void* stream);

/*
 * Dequantize b-bit codes to w_out device [n][k] bfloat16.  k <= 65536.
 * Errors: OPQ_ERR_NULL, OPQ_ERR_SHAPE, OPQ_ERR_ALPHA, OPQ_ERR_ALIGN,
 * OPQ_ERR_UNSUPPORTED, OPQ_ERR_HIP.
 */
int opq_dequantize_bits(const uint32_t* packed, const uint32_t* sign, const float* scale,
                        int64_t n, int64_t k, int bits, float alpha, uint16_t* w_out,
                        void* stream);

/*
 * opq_error_sums with b-bit codes (the same row_sums layout and precision):
 * the reconstruction error per bit width, nothing stored.  Same limits as
 * opq_quantize_bits (for bits = 4, those of opq_error_sums).
 */
int opq_error_sums_bits(const void* w, int w_dtype, int64_t n, int64_t k, int bits, float alpha,
                        double* row_sums, void* stream);

/*
 * Bytes of device workspace opq_linear_bits needs: for bits = 4 those of
 * opq_linear_workspace_bytes, otherwise room for W' as bfloat16, n * k * 2
 * bytes rounded up to 256 (0 for an empty shape).
 */
size_t opq_linear_bits_workspace_bytes(int64_t m, int64_t n, int64_t k, int bits);

/*
 * The linear layer on b-bit codes: y = x W'^T (+ bias) with W' the
 * reconstruction opq_dequantize_bits writes.  For bits = 4 this is opq_linear.
 * For 3, 5 and 6 bits the call first writes W' (bfloat16, [n][k]) into the
 * workspace with the b-bit dequantizer and then multiplies with bf16 MFMA and
 * float32 accumulation, as the card's OPQLinear decodes its weights before a
 * dense matmul ("文件结构": opq_quantize.py; "技术细节 / 推理解码").
 *   x, bias, y, y_dtype   as for opq_linear
 *   packed, sign, scale   as written by opq_quantize_bits for W[n][k]
 *   workspace, workspace_bytes  device scratch of at least
 *           opq_linear_bits_workspace_bytes(m, n, k, bits) bytes; its
 *           contents need no initialisation and are overwritten; calls that may
 *           run at the same time need buffers of their own
 * Reproducible sum order; k <= 65536, n <= 2^26.  Errors: OPQ_ERR_NULL,
 * OPQ_ERR_SHAPE (also for bits outside 3..6), OPQ_ERR_ALPHA, OPQ_ERR_ALIGN,
 * OPQ_ERR_DTYPE, OPQ_ERR_WORKSPACE, OPQ_ERR_UNSUPPORTED, OPQ_ERR_HIP.
 */
int opq_linear_bits(const uint16_t* x, const uint32_t* packed, const uint32_t* sign,
                    const float* scale, const float* bias, int64_t m, int64_t n, int64_t k, int bits,
                    float alpha, void* y, int y_dtype, void* workspace, size_t workspace_bytes,
                    void* stream);

/*
 * opq_linear_bits without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The workspace opq_linear_bits would take
 * (W' as bfloat16 for 3, 5 and 6 bits; none for 4 bits) is a fixed array that
 * the library holds on every GPU it runs on (160 MiB, kept until the process
 * ends); shapes whose opq_linear_bits_workspace_bytes exceeds 160 MiB return
 * OPQ_ERR_UNSUPPORTED.  Every call on one GPU uses that same array, so calls
 * that may overlap on one GPU (other streams or threads) race; calls in one
 * stream follow each other.  No part of the array needs to start at zero.
 * The call allocates nothing (no hipMalloc, no allocator of any library).
 * Other arguments and errors as for opq_linear_bits, plus OPQ_ERR_HIP when the
 * runtime cannot report the array's address.
 */
int opq_linear_bits_noalloc(const uint16_t* x, const uint32_t* packed, const uint32_t* sign,
                            const float* scale, const float* bias, int64_t m, int64_t n, int64_t k,
                            int bits, float alpha, void* y, int y_dtype, void* stream);

/*
 * Group-wise stored form: the card's own ("技术细节 / 存储格式": one float16
 * max per group of weights; the configuration section offers groups of 32,
 * 64, 128 or 256 weights; "推理解码": the decode multiplies by that group
 * max).  The three calls below mirror opq_quantize, opq_dequantize and
 * opq_linear with one float16 scale per group instead of one float32 scale
 * per row; packing, signs and the level table are the same.
 *   group    32, 64, 128 or 256: a group is `group` consecutive weights of a
 *            row along k; k must be a multiple of it (OPQ_ERR_SHAPE
 *            otherwise)
 *   scale16  [n][k/group] float16 bit patterns: the group's max|w| rounded to
 *            float16 (nearest, ties to even), saturated at 65504
 * Codes are taken against the stored max m16: u = |w| / m16 (binary32,
 * nearest even), q = the integer nearest to 15 u^alpha, and q = 15 whenever
 * u >= 1 (u exceeds 1 by less than 2^-11 when the max was rounded down); a
 * group whose m16 is 0 (every |w| < 2^-25) gets codes 0; sign bits are 1
 * exactly when w < 0.  Code q of a group reconstructs to bf16(G_q * m16) with
 * the sign, code 0 to +0.0.  alpha must have a separating bucket grid (every
 * alpha in [0.05, 60] has one) and keep G_1 * 2^-24 a normal binary32;
 * otherwise OPQ_ERR_UNSUPPORTED.  Other conventions as for the row form.
 */

/*
 * Quantize to the group-wise form: w device [n][k] float32 or bfloat16;
 * packed [n][k/8], sign [n][k/32], scale16 [n][k/group] device outputs.
 * Any k (a multiple of group and of 32).  Errors: OPQ_ERR_NULL, OPQ_ERR_SHAPE,
 * OPQ_ERR_ALPHA, OPQ_ERR_ALIGN, OPQ_ERR_DTYPE, OPQ_ERR_UNSUPPORTED, OPQ_ERR_HIP.
 */
int opq_quantize_grouped(const void* w, int w_dtype, int64_t n, int64_t k, int64_t group,
                         float alpha, uint32_t* packed, uint32_t* sign, uint16_t* scale16,
                         void* stream);

/*
 * Dequantize the group-wise form to w_out device [n][k] bfloat16.  Any k.
 * Errors: OPQ_ERR_NULL, OPQ_ERR_SHAPE, OPQ_ERR_ALPHA, OPQ_ERR_ALIGN,
 * OPQ_ERR_UNSUPPORTED, OPQ_ERR_HIP.
 */
int opq_dequantize_grouped(const uint32_t* packed, const uint32_t* sign, const uint16_t* scale16,
                           int64_t n, int64_t k, int64_t group, float alpha, uint16_t* w_out,
                           void* stream);

/*
 * The linear layer on the group-wise form: y = x W'^T (+ bias) with W' the
 * reconstruction opq_dequantize_grouped writes, made on chip; otherwise as
 * opq_linear (reproducible sum order, k <= 65536, n <= 2^26).  The group-wise
 * kernels use no workspace: workspace may be NULL (or any 16-byte aligned
 * pointer) and workspace_bytes any value.  Errors: OPQ_ERR_NULL,
 * OPQ_ERR_SHAPE, OPQ_ERR_ALPHA, OPQ_ERR_ALIGN, OPQ_ERR_DTYPE,
 * OPQ_ERR_UNSUPPORTED, OPQ_ERR_HIP.
 */
int opq_linear_grouped(const uint16_t* x, const uint32_t* packed, const uint32_t* sign,
                       const uint16_t* scale16, const float* bias, int64_t m, int64_t n,
                       int64_t k, int64_t group, float alpha, void* y, int y_dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* OPQ_H */
