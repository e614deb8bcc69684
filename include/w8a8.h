/*
 * w8a8.h -- C ABI of the INT8 W8A8 linear layer in libq4k (gfx950).
 *
 * Source for what is computed: "xpu-kernels -- fused kernels for Intel Arc
 * (Xe2) ...", sections "Quick start" (a bf16 [N, K] weight becomes int8 plus
 * one fp32 scale per row, once; the layer computes y = x W^T + bias), "Use
 * from C" and "API" (an int8 x int8 GEMM into int32 accumulators followed by
 * the dequant epilogue out = acc * x_scale[m] * w_scale[n] + bias[n] from
 * int32 [M, N] to bf16 [M, N]; the accumulator path that hands the int32
 * result to the caller; dequant of that accumulator reproduces the fused
 * layer bit for bit).  The page's activation quantizer also applies a
 * Kronecker-Hadamard rotation; this library does not rotate (quantize plain
 * rows, or pass codes that were rotated elsewhere).
 *
 * Layouts (row-major, no padding):
 *   x       int8 [m, k]     activation codes
 *   x_scale fp32 [m]        one scale per activation row
 *   w       int8 [n, k]     weight codes, one row per output column
 *   w_scale fp32 [n]        one scale per weight row
 *   bias    fp32 [n]        or NULL for no bias
 *   acc     int32 [m, n]    acc[i, j] = sum_c x[i, c] * w[j, c], exact
 *   out     bf16 bits [m, n]
 * Epilogue, per output: a = fp32(acc) (nearest even); a = a * x_scale[i];
 * a = a * w_scale[j]; a = a + bias[j] (skipped for NULL bias); out = bf16(a)
 * (nearest even).  Each operation is rounded on its own, in that order, never
 * fused, so w8a8_linear and w8a8_dequant_epilogue(w8a8_linear_acc(...)) give
 * identical bits.  Scales and bias must be finite; an epilogue value beyond
 * the bf16 range rounds to +-inf.
 *
 * Conventions are those of q4k.h: device pointers on the current HIP device,
 * owned by the caller; asynchronous on `stream` (NULL = the null stream);
 * int64 sizes; arguments validated before anything is enqueued, with the
 * return codes Q4K_OK / Q4K_ERR_* and the reason in q4k_last_error(); outputs
 * may not overlap inputs.  The library allocates nothing on these calls.
 */
#ifndef LIBQ4K_W8A8_H
#define LIBQ4K_W8A8_H

#include <stdint.h>

#include "q4k.h"

#ifdef __cplusplus
extern "C" {
#endif

/* k of the GEMM entry points: a positive multiple of W8A8_K_STEP, at most
 * W8A8_MAX_K (so that the largest possible sum, 128 * 128 * k, fits in int32). */
#define W8A8_K_STEP 128
#define W8A8_MAX_K 130944

/* out = bf16(acc * x_scale[m] * w_scale[n] + bias[n]) with acc = x w^T in
 * int32, in one kernel (the accumulator never leaves registers).  [xpu-kernels
 * "Use from C": the GEMM and the dequant epilogue, fused.]
 * m, n >= 1 (each at most INT32_MAX); k as above.  x, w and out 16-byte
 * aligned; x_scale, w_scale and bias 4-byte aligned.  Returns Q4K_OK,
 * Q4K_ERR_INVALID_ARG (null pointer other than bias, size out of range,
 * overlap), Q4K_ERR_ALIGN, Q4K_ERR_DEVICE or Q4K_ERR_LAUNCH. */
int w8a8_linear(const int8_t* x, const float* x_scale, const int8_t* w, const float* w_scale,
                const float* bias, uint16_t* out, int64_t m, int64_t n, int64_t k,
                void* stream);

/* acc = x w^T in int32 [m, n], exact.  [xpu-kernels "API": the accumulator
 * path.]  Sizes as w8a8_linear; x, w and acc 16-byte aligned. */
int w8a8_linear_acc(const int8_t* x, const int8_t* w, int32_t* acc, int64_t m, int64_t n,
                    int64_t k, void* stream);

/* The dequant epilogue alone: int32 [m, n] -> bf16 [m, n].  [xpu-kernels
 * "API": the dequant epilogue entry point, same argument order.]  m, n >= 1;
 * acc and out 16-byte aligned, the vectors 4-byte aligned. */
int w8a8_dequant_epilogue(const int32_t* acc, uint16_t* out, const float* x_scale,
                          const float* w_scale, const float* bias, int64_t m, int64_t n,
                          void* stream);

/* Per-row quantizer: bf16 bits [rows, k] -> int8 codes [rows, k] and fp32
 * scales [rows].  scale = amax / 127 (fp32, amax = max |v| over the row) and
 * code = clamp(rint(v / scale), -127, 127) with the division in fp32 and
 * rint rounding ties to even; a row of zeros gets scale 0 and codes 0.  Serves
 * both the one-time weight preparation and the per-call activation
 * quantization.  [xpu-kernels "Quick start": int8 plus one fp32 scale per
 * row; the page's version also rotates.]  rows >= 1, k a positive multiple of
 * 8 (at most INT32_MAX); x and q 16-byte aligned, scale 4-byte aligned;
 * inputs finite. */
int w8a8_quantize_rows(const uint16_t* x_bf16, int8_t* q, float* scale, int64_t rows,
                       int64_t k, void* stream);

#ifdef __cplusplus
}
#endif
#endif
