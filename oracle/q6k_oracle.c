/*
 * q6k_oracle.c -- plain, slow CPU oracle for Q6_K.  TEST INFRASTRUCTURE ONLY;
 * see q6k_oracle.h for the layout reading and the page it follows.  Plain
 * C11, -O2, no fast-math, -ffp-contract=off.
 */
#include "q6k_oracle.h"

#include <math.h>
#include <stdlib.h>

#include "q4k_oracle.h"

static int valid_shape(int64_t n, int64_t k) { return n >= 0 && k >= 0 && k % 256 == 0; }

int oracle_q6k_quant(const uint8_t blk[210], int i) {
  const int h = i / 128, j = (i / 32) % 4, l = i % 32;
  const uint8_t lo = blk[64 * h + 32 * (j % 2) + l];
  const int nibble = j < 2 ? (lo & 15) : (lo >> 4);
  const int high = (blk[128 + 32 * h + l] >> (2 * j)) & 3;
  return nibble + 16 * high;
}

void oracle_q6k_dequant_block(const uint8_t blk[210], float w[256]) {
  const double d = oracle_f16_to_f64((uint16_t)(blk[208] | (blk[209] << 8)));
  for (int i = 0; i < 256; ++i) {
    const int sc = (int8_t)blk[192 + i / 16];
    /* exact in fp64 (at most 24 significant bits), then one rounding */
    w[i] = (float)(d * (double)sc * (double)(oracle_q6k_quant(blk, i) - 32));
  }
}

static void dequant_row(const uint8_t *w, int64_t r, int64_t k, float *row) {
  const int64_t nb = k / 256;
  for (int64_t b = 0; b < nb; ++b)
    oracle_q6k_dequant_block(w + (r * nb + b) * ORACLE_Q6K_BLOCK_BYTES, row + 256 * b);
}

int oracle_q6k_dequant_f32(const uint8_t *w, int64_t n, int64_t k, float *out) {
  if (!valid_shape(n, k)) return -1;
  for (int64_t r = 0; r < n; ++r) dequant_row(w, r, k, out + r * k);
  return 0;
}

int oracle_q6k_dequant_bf16(const uint8_t *w, int64_t n, int64_t k, uint16_t *out) {
  if (!valid_shape(n, k)) return -1;
  float *row = (float *)malloc((size_t)(k > 0 ? k : 1) * sizeof(float));
  if (!row) return -1;
  for (int64_t r = 0; r < n; ++r) {
    dequant_row(w, r, k, row);
    for (int64_t c = 0; c < k; ++c) out[r * k + c] = oracle_f32_to_bf16(row[c]);
  }
  free(row);
  return 0;
}

/* y[i, j] = sum_k W[j, k] x[i, k] with exact fp64 products summed in k order;
 * a = sum |W x| (the tolerance scale). */
int oracle_q6k_gemv_rows(const uint8_t *w, const float *x, int64_t m, int64_t n,
                         int64_t k, const int64_t *rows, int64_t nrows,
                         double *y, double *a) {
  if (!valid_shape(n, k) || m < 0 || nrows < 0) return -1;
  for (int64_t t = 0; t < nrows; ++t)
    if (rows[t] < 0 || rows[t] >= n) return -1;
  float *wrow = (float *)malloc((size_t)(k > 0 ? k : 1) * sizeof(float));
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

int oracle_q6k_gemv(const uint8_t *w, const float *x, int64_t m, int64_t n,
                    int64_t k, double *y, double *a) {
  if (!valid_shape(n, k) || m < 0) return -1;
  int64_t *rows = (int64_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(int64_t));
  if (!rows) return -1;
  for (int64_t j = 0; j < n; ++j) rows[j] = j;
  const int rc = oracle_q6k_gemv_rows(w, x, m, n, k, rows, n, y, a);
  free(rows);
  return rc;
}

/* Y[i, j] = sum_c X[i, c] W[j, c] with X decoded exactly from bf16; each
 * product is exact in fp64, summed in c order. */
int oracle_q6k_gemm_cols(const uint8_t *w, const uint16_t *x, int64_t m, int64_t n,
                         int64_t k, const int64_t *cols, int64_t ncols,
                         double *y, double *a) {
  if (!valid_shape(n, k) || m < 0 || ncols < 0) return -1;
  for (int64_t t = 0; t < ncols; ++t)
    if (cols[t] < 0 || cols[t] >= n) return -1;
  float *wrow = (float *)malloc((size_t)(k > 0 ? k : 1) * sizeof(float));
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

int oracle_q6k_gemm(const uint8_t *w, const uint16_t *x, int64_t m, int64_t n,
                    int64_t k, double *y, double *a) {
  if (!valid_shape(n, k) || m < 0) return -1;
  int64_t *cols = (int64_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(int64_t));
  if (!cols) return -1;
  for (int64_t j = 0; j < n; ++j) cols[j] = j;
  const int rc = oracle_q6k_gemm_cols(w, x, m, n, k, cols, n, y, a);
  free(cols);
  return rc;
}
