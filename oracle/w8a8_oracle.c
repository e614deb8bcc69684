/*
 * w8a8_oracle.c -- plain, slow CPU oracle for the INT8 W8A8 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY; see w8a8_oracle.h for the passage it follows and
 * the reading of the epilogue.  Build: plain C11, -O2, no fast-math and
 * -ffp-contract=off, so every fp32 operation below rounds on its own.
 */
#include "w8a8_oracle.h"

#include <math.h>
#include <stdlib.h>

#include "q4k_oracle.h"

int oracle_w8a8_acc(const int8_t *x, const int8_t *w, int64_t m, int64_t n, int64_t k,
                    int32_t *acc) {
  if (m < 0 || n < 0 || k < 0) return -1;
  for (int64_t i = 0; i < m; ++i) {
    for (int64_t j = 0; j < n; ++j) {
      int64_t s = 0;
      for (int64_t c = 0; c < k; ++c) s += (int64_t)x[i * k + c] * (int64_t)w[j * k + c];
      if (s < INT32_MIN || s > INT32_MAX) return -1;
      acc[i * n + j] = (int32_t)s;
    }
  }
  return 0;
}

int oracle_w8a8_epilogue(const int32_t *acc, const float *x_scale, const float *w_scale,
                         const float *bias, int64_t m, int64_t n, uint16_t *out,
                         float *out_f32) {
  if (m < 0 || n < 0) return -1;
  for (int64_t i = 0; i < m; ++i) {
    for (int64_t j = 0; j < n; ++j) {
      volatile float a = (float)acc[i * n + j]; /* int32 -> fp32, nearest even */
      a = a * x_scale[i];
      a = a * w_scale[j];
      if (bias) a = a + bias[j];
      out[i * n + j] = oracle_f32_to_bf16(a);
      if (out_f32) out_f32[i * n + j] = a;
    }
  }
  return 0;
}

int oracle_w8a8_linear(const int8_t *x, const float *x_scale, const int8_t *w,
                       const float *w_scale, const float *bias, int64_t m, int64_t n,
                       int64_t k, uint16_t *out) {
  if (m < 0 || n < 0 || k < 0) return -1;
  int32_t *acc = (int32_t *)malloc((size_t)(m * n > 0 ? m * n : 1) * sizeof(int32_t));
  if (!acc) return -1;
  int rc = oracle_w8a8_acc(x, w, m, n, k, acc);
  if (rc == 0) rc = oracle_w8a8_epilogue(acc, x_scale, w_scale, bias, m, n, out, NULL);
  free(acc);
  return rc;
}

int oracle_w8a8_linear_cols(const int8_t *x, const float *x_scale, const int8_t *w,
                            const float *w_scale, const float *bias, int64_t m, int64_t n,
                            int64_t k, const int64_t *cols, int64_t ncols, uint16_t *out) {
  if (m < 0 || n < 0 || k < 0 || ncols < 0) return -1;
  for (int64_t c = 0; c < ncols; ++c)
    if (cols[c] < 0 || cols[c] >= n) return -1;
  for (int64_t i = 0; i < m; ++i) {
    for (int64_t c = 0; c < ncols; ++c) {
      const int64_t j = cols[c];
      int32_t acc;
      if (oracle_w8a8_acc(x + i * k, w + j * k, 1, 1, k, &acc) != 0) return -1;
      const float one_bias = bias ? bias[j] : 0.0f;
      if (oracle_w8a8_epilogue(&acc, x_scale + i, w_scale + j, bias ? &one_bias : NULL, 1, 1,
                               out + i * ncols + c, NULL) != 0)
        return -1;
    }
  }
  return 0;
}

int oracle_w8a8_quantize_rows(const uint16_t *x, int64_t rows, int64_t k, int8_t *q,
                              float *scale) {
  if (rows < 0 || k < 0) return -1;
  for (int64_t r = 0; r < rows; ++r) {
    const uint16_t *row = x + r * k;
    float amax = 0.0f;
    for (int64_t c = 0; c < k; ++c) {
      const float v = fabsf((float)oracle_bf16_to_f64(row[c])); /* exact */
      if (v > amax) amax = v;
    }
    volatile float s = amax / 127.0f;
    scale[r] = s;
    for (int64_t c = 0; c < k; ++c) {
      if (s == 0.0f) {
        q[r * k + c] = 0;
        continue;
      }
      volatile float v = (float)oracle_bf16_to_f64(row[c]) / s;
      float t = rintf(v); /* nearest integer, ties to even (default rounding mode) */
      if (t > 127.0f) t = 127.0f;
      if (t < -127.0f) t = -127.0f;
      q[r * k + c] = (int8_t)t;
    }
  }
  return 0;
}
