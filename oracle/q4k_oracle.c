/*
 * q4k_oracle.c -- plain, slow CPU oracle for the Q4_K linear layer.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU-baseline leg; never by the product path.  It shares no code
 * with the HIP library.  See q4k_oracle.h for the sources it follows and the
 * arithmetic it fixes.
 *
 * Build: plain C11, -O2, no fast-math and -ffp-contract=off, so every
 * operation below is evaluated exactly as written.
 */
#include "q4k_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- binary16 -------------------------------------------------------------
 * IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Exponent 0 encodes zero and subnormals (value = f * 2^-24); exponent 31
 * encodes infinities and NaNs.  The super-block scales d and dmin are fp16
 * ("Writing an ESIMD Fused Kernel ...", "Getting Q4_K Right", and the format
 * reading); subnormal scales are kept, never flushed. */
double oracle_f16_to_f64(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int e = (h >> 10) & 0x1f;
  const int f = h & 0x3ff;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24);
  } else if (e == 31) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + f), e - 25);
  }
  return sign ? -v : v;
}

float oracle_f16_to_f32(uint16_t h) { return (float)oracle_f16_to_f64(h); }

/* ---- 6-bit scales and mins ------------------------------------------------
 * Format reading (the pages name "6-bit sub-block scales and mins" but print
 * no packing): 12 bytes s[0..11] hold sc[0..7] and mn[0..7].
 *   sub-blocks 0..3: sc[j] = low 6 bits of s[j],   mn[j] = low 6 bits of s[j+4]
 *   sub-blocks 4..7: sc[j] = low nibble of s[j+4], plus the top 2 bits of
 *                    s[j-4] as bits 4..5;
 *                    mn[j] = high nibble of s[j+4], plus the top 2 bits of
 *                    s[j] as bits 4..5. */
void oracle_unpack_scales(const uint8_t s[12], uint8_t sc[8], uint8_t mn[8]) {
  for (int j = 0; j < 4; ++j) {
    sc[j] = (uint8_t)(s[j] % 64);
    mn[j] = (uint8_t)(s[j + 4] % 64);
  }
  for (int j = 4; j < 8; ++j) {
    const int lo_sc = s[j + 4] % 16;
    const int lo_mn = s[j + 4] / 16;
    const int hi_sc = s[j - 4] / 64;
    const int hi_mn = s[j] / 64;
    sc[j] = (uint8_t)(lo_sc + 16 * hi_sc);
    mn[j] = (uint8_t)(lo_mn + 16 * hi_mn);
  }
}

/* ---- 4-bit quants -----------------------------------------------------------
 * Format reading of the "y-offset mapping" ("Getting Q4_K Right"): the 128
 * quant bytes form four groups of 32.  In group g, the low nibble of byte
 * 32g + r is weight 64g + r and the high nibble is weight 64g + 32 + r, for
 * r = 0..31.  Sub-block j covers weights 32j .. 32j + 31. */
int oracle_quant(const uint8_t qs[128], int i) {
  const int g = i / 64;
  const int r = i % 64;
  if (r < 32) return qs[32 * g + r] % 16;
  return qs[32 * g + (r - 32)] / 16;
}

/* ---- dequantization ---------------------------------------------------------
 * w_i = d * sc[j] * q_i - dmin * mn[j], j = i / 32.  Evaluated in fp64, where
 * both products and their difference are exact (fp16 scales times integers
 * below 2^10 span fewer than 53 bits), then rounded once to fp32. */
void oracle_dequant_block(const uint8_t blk[144], float w[256]) {
  const uint16_t d_bits = (uint16_t)(blk[0] | (blk[1] << 8));
  const uint16_t dmin_bits = (uint16_t)(blk[2] | (blk[3] << 8));
  const double d = oracle_f16_to_f64(d_bits);
  const double dmin = oracle_f16_to_f64(dmin_bits);
  uint8_t sc[8], mn[8];
  oracle_unpack_scales(blk + 4, sc, mn);
  const uint8_t *qs = blk + 16;
  for (int i = 0; i < 256; ++i) {
    const int j = i / 32;
    const double scaled = d * (double)sc[j] * (double)oracle_quant(qs, i);
    const double offset = dmin * (double)mn[j];
    w[i] = (float)(scaled - offset);
  }
}

static int valid_shape(int64_t n, int64_t k) {
  return n >= 0 && k > 0 && k % ORACLE_QK == 0;
}

/* Row r of W: k/256 consecutive blocks at byte offset r * (k/256) * 144. */
static void dequant_row(const uint8_t *w, int64_t r, int64_t k, float *out) {
  const int64_t nb = k / ORACLE_QK;
  for (int64_t b = 0; b < nb; ++b) {
    oracle_dequant_block(w + (r * nb + b) * ORACLE_BLOCK_BYTES, out + b * ORACLE_QK);
  }
}

int oracle_dequant_f32(const uint8_t *w, int64_t n, int64_t k, float *out) {
  if (!valid_shape(n, k)) return -1;
  for (int64_t r = 0; r < n; ++r) dequant_row(w, r, k, out + r * k);
  return 0;
}

/* bf16 keeps the top 16 bits of the fp32 pattern; round to nearest, ties to
 * even, by adding 0x7fff plus the lowest kept bit before truncating. */
uint16_t oracle_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) {
    return (uint16_t)((u >> 16) | 0x40u); /* quiet NaN */
  }
  const uint32_t lsb = (u >> 16) & 1u;
  return (uint16_t)((u + 0x7fffu + lsb) >> 16);
}

double oracle_bf16_to_f64(uint16_t b) {
  const uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

int oracle_dequant_bf16(const uint8_t *w, int64_t n, int64_t k, uint16_t *out) {
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

/* ---- GEMV ---------------------------------------------------------------------
 * y[i, j] = sum_k W[j, k] x[i, k]: the linear layer at decode, weights
 * dequantized then dotted ("Getting Q4_K Right": dequant plus a dot product).
 * Each fp32 x fp32 product is exact in fp64; the sum runs in k order. */
static void dot_row(const float *wrow, const float *xrow, int64_t k, double *y,
                    double *a) {
  double s = 0.0, t = 0.0;
  for (int64_t c = 0; c < k; ++c) {
    const double p = (double)wrow[c] * (double)xrow[c];
    s += p;
    t += fabs(p);
  }
  *y = s;
  *a = t;
}

/* Output rows are independent: in the OpenMP build (liboracle_omp.so, the
 * benchmark's all-cores CPU baseline) threads take whole rows, each summed in
 * the same k order, so both builds return identical bits.  The plain build
 * ignores the pragmas and runs the loop as written. */
int oracle_gemv_rows(const uint8_t *w, const float *x, int64_t m, int64_t n,
                     int64_t k, const int64_t *rows, int64_t nrows, double *y,
                     double *a) {
  if (!valid_shape(n, k) || m < 0 || nrows < 0) return -1;
  for (int64_t t = 0; t < nrows; ++t) {
    if (rows[t] < 0 || rows[t] >= n) return -1;
  }
  int rc = 0;
#pragma omp parallel
  {
    float *wrow = (float *)malloc((size_t)k * sizeof(float));
    if (!wrow) {
#pragma omp atomic write
      rc = -1;
    }
#pragma omp for schedule(static)
    for (int64_t t = 0; t < nrows; ++t) {
      if (!wrow) continue;
      dequant_row(w, rows[t], k, wrow);
      for (int64_t i = 0; i < m; ++i) {
        dot_row(wrow, x + i * k, k, &y[i * nrows + t], &a[i * nrows + t]);
      }
    }
    free(wrow);
  }
  return rc;
}

int oracle_gemv(const uint8_t *w, const float *x, int64_t m, int64_t n,
                int64_t k, double *y, double *a) {
  if (!valid_shape(n, k) || m < 0) return -1;
  int64_t *rows = (int64_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(int64_t));
  if (!rows) return -1;
  for (int64_t j = 0; j < n; ++j) rows[j] = j;
  const int rc = oracle_gemv_rows(w, x, m, n, k, rows, n, y, a);
  free(rows);
  return rc;
}

/* ---- GEMM ---------------------------------------------------------------------
 * Y[i, j] = sum_k X[i, k] W[j, k] with X in bf16 (the prefill tile GEMM).
 * The oracle uses the fp32 dequantized weights; bf16 x fp32 products are exact
 * in fp64. */
int oracle_gemm_cols(const uint8_t *w, const uint16_t *x, int64_t m, int64_t n,
                     int64_t k, const int64_t *cols, int64_t ncols, double *y,
                     double *a) {
  if (!valid_shape(n, k) || m < 0 || ncols < 0) return -1;
  for (int64_t t = 0; t < ncols; ++t) {
    if (cols[t] < 0 || cols[t] >= n) return -1;
  }
  int rc = 0;
#pragma omp parallel
  {
    float *wrow = (float *)malloc((size_t)k * sizeof(float));
    if (!wrow) {
#pragma omp atomic write
      rc = -1;
    }
#pragma omp for schedule(static)
    for (int64_t t = 0; t < ncols; ++t) {
      if (!wrow) continue;
      dequant_row(w, cols[t], k, wrow);
      for (int64_t i = 0; i < m; ++i) {
        double s = 0.0, u = 0.0;
        const uint16_t *xrow = x + i * k;
        for (int64_t c = 0; c < k; ++c) {
          const double p = oracle_bf16_to_f64(xrow[c]) * (double)wrow[c];
          s += p;
          u += fabs(p);
        }
        y[i * ncols + t] = s;
        a[i * ncols + t] = u;
      }
    }
    free(wrow);
  }
  return rc;
}

int oracle_gemm(const uint8_t *w, const uint16_t *x, int64_t m, int64_t n,
                int64_t k, double *y, double *a) {
  if (!valid_shape(n, k) || m < 0) return -1;
  int64_t *cols = (int64_t *)malloc((size_t)(n > 0 ? n : 1) * sizeof(int64_t));
  if (!cols) return -1;
  for (int64_t j = 0; j < n; ++j) cols[j] = j;
  const int rc = oracle_gemm_cols(w, x, m, n, k, cols, n, y, a);
  free(cols);
  return rc;
}

/* ---- SwiGLU MLP ------------------------------------------------------------------
 * The MUL_MAT + MUL_MAT + SWIGLU pattern ("Building ESIMD Infrastructure"):
 * gate and up projections of the same x, h = silu(gate) * up, then the down
 * projection of h.  silu is the textbook t * sigmoid(t). */
double oracle_silu(double t) { return t / (1.0 + exp(-t)); }

/* Threads the row loops use: 1 in the plain build, the OpenMP team size in the
 * OpenMP build. */
int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

int oracle_swiglu_mlp(const uint8_t *w_gate, const uint8_t *w_up,
                      const uint8_t *w_down, const float *x, int64_t d_model,
                      int64_t d_ff, double *g, double *ag, double *u,
                      double *au, double *h, double *out, double *aout) {
  if (!valid_shape(d_ff, d_model) || !valid_shape(d_model, d_ff) || !out) return -1;
  const size_t nf = (size_t)d_ff;
  double *gg = (double *)malloc(nf * sizeof(double));
  double *ga = (double *)malloc(nf * sizeof(double));
  double *uu = (double *)malloc(nf * sizeof(double));
  double *ua = (double *)malloc(nf * sizeof(double));
  double *hh = (double *)malloc(nf * sizeof(double));
  int rc = -1;
  if (!gg || !ga || !uu || !ua || !hh) goto done;
  if (oracle_gemv(w_gate, x, 1, d_ff, d_model, gg, ga)) goto done;
  if (oracle_gemv(w_up, x, 1, d_ff, d_model, uu, ua)) goto done;
  for (int64_t f = 0; f < d_ff; ++f) hh[f] = oracle_silu(gg[f]) * uu[f];
#pragma omp parallel
  {
    float *drow = (float *)malloc((size_t)d_ff * sizeof(float));
#pragma omp for schedule(static)
    for (int64_t r = 0; r < d_model; ++r) {
      if (!drow) continue;
      dequant_row(w_down, r, d_ff, drow);
      double s = 0.0, t = 0.0;
      for (int64_t f = 0; f < d_ff; ++f) {
        const double p = (double)drow[f] * hh[f];
        s += p;
        t += fabs(p);
      }
      out[r] = s;
      if (aout) aout[r] = t;
    }
    if (!drow) {
#pragma omp atomic write
      rc = -2;
    }
    free(drow);
  }
  if (rc == -2) goto done;
  if (g) memcpy(g, gg, nf * sizeof(double));
  if (ag) memcpy(ag, ga, nf * sizeof(double));
  if (u) memcpy(u, uu, nf * sizeof(double));
  if (au) memcpy(au, ua, nf * sizeof(double));
  if (h) memcpy(h, hh, nf * sizeof(double));
  rc = 0;
done:
  free(gg);
  free(ga);
  free(uu);
  free(ua);
  free(hh);
  return rc;
}
