/*
 * w8a8_oracle.h -- plain, slow CPU oracle for the INT8 W8A8 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY, like q4k_oracle.h: only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it; it shares no code
 * with the HIP library.
 *
 * Source: "xpu-kernels -- fused kernels for Intel Arc (Xe2) ...", sections
 * "API" and "Use from C": an int8 x int8 GEMM into int32 accumulators
 * (activations int8 [M, K] with one fp32 scale per row, weights int8 [N, K]
 * with one fp32 scale per row) and the dequant epilogue
 *   out = acc * x_scale[m] * w_scale[n] + bias[n]   (int32 [M, N] -> bf16).
 * The activation rotation that the page pairs with the quantizer is out of
 * scope; inputs arrive already quantized.
 *
 * Reading of the epilogue (the page gives the expression only): evaluated
 * left to right in fp32, every operation rounded to nearest even and none
 * fused: a = fp32(acc); a = a * x_scale[m]; a = a * w_scale[n];
 * a = a + bias[n] (skipped when bias is NULL); out = bf16 nearest even of a.
 *
 * Row quantizer (the same page, "Quick start": the weight is turned into int8
 * plus one fp32 scale per output row once, and the activation into int8 plus
 * one fp32 scale per row; the page's quantizer also rotates, which is out of
 * scope here).  Reading: per row, amax = max |v| over the row (bf16 inputs
 * widened exactly to fp32), scale = amax / 127 in fp32, and each code is
 * v / scale in fp32, rounded to the nearest integer with ties to even and
 * clamped to [-127, 127].  A row of zeros gets scale 0 and codes 0.  Inputs
 * must be finite.
 *
 * Errors: 0 on success; -1 for a bad size or an accumulator outside int32.
 */
#ifndef W8A8_ORACLE_H
#define W8A8_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* acc[i, j] = sum_c x[i, c] * w[j, c], exact (int64), stored as int32. */
int oracle_w8a8_acc(const int8_t *x, const int8_t *w, int64_t m, int64_t n, int64_t k,
                    int32_t *acc);

/* The epilogue on given accumulators: out bf16 bits [m, n] (and, if out_f32 is
 * not NULL, the fp32 value before the bf16 rounding). */
int oracle_w8a8_epilogue(const int32_t *acc, const float *x_scale, const float *w_scale,
                         const float *bias, int64_t m, int64_t n, uint16_t *out,
                         float *out_f32);

/* acc then the epilogue. */
int oracle_w8a8_linear(const int8_t *x, const float *x_scale, const int8_t *w,
                       const float *w_scale, const float *bias, int64_t m, int64_t n,
                       int64_t k, uint16_t *out);

/* acc then the epilogue, for the output columns cols[0..ncols) only:
 * out bf16 bits [m, ncols]. */
int oracle_w8a8_linear_cols(const int8_t *x, const float *x_scale, const int8_t *w,
                            const float *w_scale, const float *bias, int64_t m, int64_t n,
                            int64_t k, const int64_t *cols, int64_t ncols, uint16_t *out);

/* Row quantizer: x bf16 bits [rows, k] -> q int8 [rows, k], scale fp32 [rows]. */
int oracle_w8a8_quantize_rows(const uint16_t *x, int64_t rows, int64_t k, int8_t *q,
                              float *scale);

#ifdef __cplusplus
}
#endif
#endif
