/*
 * q4k_oracle.h -- plain, slow CPU oracle for the Q4_K linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library libq4k and its Python binding) never calls it, links it or
 * falls back to it, and it shares no code, header, table or constant with
 * that path.
 *
 * What it computes (sources, by page title and section):
 *   - "Writing an ESIMD Fused Kernel From Reverse-Engineered Assembly",
 *     section "Getting Q4_K Right": Q4_K super-block dequantization followed
 *     by a dot product; section "Building ESIMD Infrastructure": the
 *     MUL_MAT + MUL_MAT + SWIGLU MLP pattern.
 *   - "CPU kernel parity: decode and tile kernels at llama.cpp speed ..."
 *     (daScript PR page), section "Validation": every kernel variant must be
 *     bit-exact against the reference decode.
 *   - "xpu-kernels -- fused kernels for Intel Arc (Xe2) ...", section
 *     "Algorithm: fused ConvRot rotation": results are checked against a
 *     float64 ground truth on the CPU.
 *
 * The pages print no byte layout for a Q4_K super-block.  The layout used
 * here is the reading documented with the project (144 bytes: fp16 d at 0,
 * fp16 dmin at 2, twelve bytes of packed 6-bit scales/mins at 4, 128 bytes of
 * 4-bit quants at 16); every function below that depends on it says so.
 *
 * Arithmetic: dequantization is done in fp64 and rounded once to fp32 (the
 * exact result rounded to nearest-even); dot products accumulate the exact
 * fp64 products of the fp32 weights and fp32 (or bf16) activations in fp64,
 * in increasing k order.  Besides each result the oracle returns
 * A = sum_k |w*x| in fp64, the scale of the parity tolerances.
 *
 * Errors: every int-returning function returns 0 on success and -1 on an
 * invalid size (k not a positive multiple of 256, negative counts, index out
 * of range).  Nothing is allocated that the caller does not see freed before
 * return.
 */
#ifndef Q4K_ORACLE_H
#define Q4K_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weights per super-block and bytes per super-block (reading of the format). */
enum { ORACLE_QK = 256, ORACLE_BLOCK_BYTES = 144 };

/* IEEE binary16 (little-endian bit pattern) -> value, subnormals kept. */
double oracle_f16_to_f64(uint16_t h);
float oracle_f16_to_f32(uint16_t h);

/* Eight 6-bit scales sc[] and eight 6-bit mins mn[] from the 12 packed bytes. */
void oracle_unpack_scales(const uint8_t s[12], uint8_t sc[8], uint8_t mn[8]);

/* 4-bit quant of weight i (0..255) of a block from its 128 quant bytes. */
int oracle_quant(const uint8_t qs[128], int i);

/* One 144-byte super-block -> 256 fp32 weights. */
void oracle_dequant_block(const uint8_t blk[144], float w[256]);

/* W [n, k] in Q4_K (n rows of k/256 blocks) -> fp32 [n, k] / bf16 bits [n, k]. */
int oracle_dequant_f32(const uint8_t *w, int64_t n, int64_t k, float *out);
int oracle_dequant_bf16(const uint8_t *w, int64_t n, int64_t k, uint16_t *out);

/* fp32 -> bf16 bit pattern, round to nearest even (NaN stays NaN). */
uint16_t oracle_f32_to_bf16(float f);
/* bf16 bit pattern -> value (exact). */
double oracle_bf16_to_f64(uint16_t b);

/* GEMV: y[i, j] = sum_k W[j, k] * x[i, k] for i < m, j < n, with x fp32
 * [m, k] row-major; y and a are fp64 [m, n] row-major. */
int oracle_gemv(const uint8_t *w, const float *x, int64_t m, int64_t n,
                int64_t k, double *y, double *a);

/* Same, only for the output columns rows[0..nrows): y, a are [m, nrows]. */
int oracle_gemv_rows(const uint8_t *w, const float *x, int64_t m, int64_t n,
                     int64_t k, const int64_t *rows, int64_t nrows, double *y,
                     double *a);

/* GEMM: Y[i, j] = sum_k X[i, k] * W[j, k] with X bf16 bits [m, k]; Y, A fp64
 * [m, n].  The weights are the fp32 dequantized values (not bf16-rounded). */
int oracle_gemm(const uint8_t *w, const uint16_t *x, int64_t m, int64_t n,
                int64_t k, double *y, double *a);

/* Same, only for the output columns cols[0..ncols): Y, A are [m, ncols]. */
int oracle_gemm_cols(const uint8_t *w, const uint16_t *x, int64_t m, int64_t n,
                     int64_t k, const int64_t *cols, int64_t ncols, double *y,
                     double *a);

/* silu(t) = t / (1 + exp(-t)), in fp64. */
double oracle_silu(double t);

/* SwiGLU MLP at one token:
 *   g = W_gate x, u = W_up x           (W_gate, W_up: [d_ff, d_model])
 *   h = silu(g) * u                    (fp64, not rounded)
 *   out = W_down h                     (W_down: [d_model, d_ff])
 * g, ag, u, au, h are fp64 [d_ff]; out, aout are fp64 [d_model], where
 * aout = sum |w_down * h|.  Any of the optional outputs may be NULL except
 * out. */
int oracle_swiglu_mlp(const uint8_t *w_gate, const uint8_t *w_up,
                      const uint8_t *w_down, const float *x, int64_t d_model,
                      int64_t d_ff, double *g, double *ag, double *u,
                      double *au, double *h, double *out, double *aout);

/* Threads the GEMV, GEMM and MLP row loops run on: 1 for liboracle.so; for
 * liboracle_omp.so (the same source built with OpenMP, used only to time the
 * oracle on all host cores) the OpenMP team size.  Both builds return
 * identical results: each output row is summed in the same order. */
int oracle_threads(void);

#ifdef __cplusplus
}
#endif
#endif
