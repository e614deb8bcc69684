/*
 * q5k_oracle.c -- plain, slow CPU oracle for the Q5_K sibling format.
 *
 * TEST INFRASTRUCTURE ONLY; see q5k_oracle.h for the format reading and the
 * passage it follows.  The fp16 decode, the 6-bit scale unpacking, the 4-bit
 * nibble map and the bf16 rounding are the Q4_K oracle's (q4k_oracle.c),
 * which this file calls; the format adds one high bit per weight.
 *
 * Build: plain C11, -O2, no fast-math and -ffp-contract=off.
 */
#include "q5k_oracle.h"

#include <math.h>
#include <stdlib.h>

#include "q4k_oracle.h"

/* Fifth bit of weight i = 64g + r: bit (2g + (r >= 32)) of qh[r mod 32]. */
int oracle_q5k_quant(const uint8_t qh[32], const uint8_t qs[128], int i) {
  const int g = i / 64;
  const int r = i % 64;
  const int bit = 2 * g + (r >= 32 ? 1 : 0);
  const int high = (qh[r % 32] >> bit) % 2;
  return oracle_quant(qs, i) + 16 * high;
}

/* w_i = d * sc[j] * q_i - dmin * mn[j] in fp64 (exact: q_i < 32, sc < 64),
 * rounded once to fp32. */
void oracle_q5k_dequant_block(const uint8_t blk[176], float w[256]) {
  const double d = oracle_f16_to_f64((uint16_t)(blk[0] | (blk[1] << 8)));
  const double dmin = oracle_f16_to_f64((uint16_t)(blk[2] | (blk[3] << 8)));
  uint8_t sc[8], mn[8];
  oracle_unpack_scales(blk + 4, sc, mn);
  const uint8_t *qh = blk + 16;
  const uint8_t *qs = blk + 48;
  for (int i = 0; i < 256; ++i) {
    const int j = i / 32;
    const double scaled = d * (double)sc[j] * (double)oracle_q5k_quant(qh, qs, i);
    const double offset = dmin * (double)mn[j];
    w[i] = (float)(scaled - offset);
  }
}

static int valid_shape(int64_t n, int64_t k) {
  return n >= 0 && k > 0 && k % ORACLE_QK == 0;
}

static void dequant_row(const uint8_t *w, int64_t r, int64_t k, float *out) {
  const int64_t nb = k / ORACLE_QK;
  for (int64_t b = 0; b < nb; ++b) {
    oracle_q5k_dequant_block(w + (r * nb + b) * ORACLE_Q5K_BLOCK_BYTES, out + b * ORACLE_QK);
  }
}

int oracle_q5k_dequant_f32(const uint8_t *w, int64_t n, int64_t k, float *out) {
  if (!valid_shape(n, k)) return -1;
  for (int64_t r = 0; r < n; ++r) dequant_row(w, r, k, out + r * k);
  return 0;
}

int oracle_q5k_dequant_bf16(const uint8_t *w, int64_t n, int64_t k, uint16_t *out) {
  if (!valid_shape(n, k)) return -1;
  float *row = (float *)malloc((size_t)k * sizeof(float));
  if (!row) return -1;
  for (int64_t r = 0; r < n; ++r) {
    dequant_row(w, r, k, row);
    for (int64_t c = 0; c < k; ++c) out[r * k + c] = oracle_f32_to_bf16(row[c]);
  }
  free(row);
  return 0;
}

/* y[i, j] = sum_k W[j, k] x[i, k] with exact fp64 products summed in k order. */
int oracle_q5k_gemv_rows(const uint8_t *w, const float *x, int64_t m, int64_t n,
                         int64_t k, const int64_t *rows, int64_t nrows,
                         double *y, double *a) {
  if (!valid_shape(n, k) || m < 0 || nrows < 0) return -1;
  for (int64_t t = 0; t < nrows; ++t) {
    if (rows[t] < 0 || rows[t] >= n) return -1;
  }
  float *wrow = (float *)malloc((size_t)k * sizeof(float));
  if (!wrow) return -1;
  for (int64_t t = 0; t < nrows; ++t) {
    dequant_row(w, rows[t], k, wrow);
    for (int64_t i = 0; i < m; ++i) {
      double s = 0.0, u = 0.0;
      for (int64_t c = 0; c < k; ++c) {
        const double p = (double)wrow[c] * (double)x[i * k + c];
        s += p;
        u += fabs(p);
      }
      y[i * nrows + t] = s;
      a[i * nrows + t] = u;
    }
  }
  free(wrow);
  return 0;
}

int oracle_q5k_gemv(const uint8_t *w, const float *x, int64_t m, int64_t n,
                    int64_t k, double *y, double *a) {
  if (!valid_shape(n, k) || m < 0) return -1;
  int64_t *rows = (int64_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(int64_t));
  if (!rows) return -1;
  for (int64_t j = 0; j < n; ++j) rows[j] = j;
  const int rc = oracle_q5k_gemv_rows(w, x, m, n, k, rows, n, y, a);
  free(rows);
  return rc;
}

/* Y[i, j] = sum_k X[i, k] W[j, k] with X in bf16 and the fp32 dequantized
 * weights (the prefill tile GEMM); bf16 x fp32 products are exact in fp64. */
int oracle_q5k_gemm_cols(const uint8_t *w, const uint16_t *x, int64_t m, int64_t n,
                         int64_t k, const int64_t *cols, int64_t ncols, double *y,
                         double *a) {
  if (!valid_shape(n, k) || m < 0 || ncols < 0) return -1;
  for (int64_t t = 0; t < ncols; ++t) {
    if (cols[t] < 0 || cols[t] >= n) return -1;
  }
  float *wrow = (float *)malloc((size_t)k * sizeof(float));
  if (!wrow) return -1;
  for (int64_t t = 0; t < ncols; ++t) {
    dequant_row(w, cols[t], k, wrow);
    for (int64_t i = 0; i < m; ++i) {
      double s = 0.0, u = 0.0;
      for (int64_t c = 0; c < k; ++c) {
        const double p = oracle_bf16_to_f64(x[i * k + c]) * (double)wrow[c];
        s += p;
        u += fabs(p);
      }
      y[i * ncols + t] = s;
      a[i * ncols + t] = u;
    }
  }
  free(wrow);
  return 0;
}

int oracle_q5k_gemm(const uint8_t *w, const uint16_t *x, int64_t m, int64_t n,
                    int64_t k, double *y, double *a) {
  if (!valid_shape(n, k) || m < 0) return -1;
  int64_t *cols = (int64_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(int64_t));
  if (!cols) return -1;
  for (int64_t j = 0; j < n; ++j) cols[j] = j;
  const int rc = oracle_q5k_gemm_cols(w, x, m, n, k, cols, n, y, a);
  free(cols);
  return rc;
}
