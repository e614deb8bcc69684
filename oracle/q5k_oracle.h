/*
 * q5k_oracle.h -- plain, slow CPU oracle for the Q5_K sibling format.
 *
 * TEST INFRASTRUCTURE ONLY, like q4k_oracle.h: only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it; it shares no code
 * with the HIP library.
 *
 * Source: "CPU kernel parity: decode and tile kernels at llama.cpp speed ..."
 * (daScript PR page), section on the kernel work: the 4-bit and 5-bit
 * k-quants ("k4", "k5") are decoded by the same fused dequant-and-dot kernel
 * shape.  The pages print no Q5_K layout.  The reading used here is the GGUF convention, the
 * Q4_K super-block plus one high bit per weight:
 *   176 bytes = fp16 d at 0, fp16 dmin at 2, the 12 packed 6-bit scale/min
 *   bytes of Q4_K at 4, 32 high-bit bytes qh at 16, 128 nibble bytes qs at 48.
 *   Weight i = 64g + r (r = 0..63): the nibble is Q4_K's (low nibble of
 *   qs[32g + r] for r < 32, high nibble of qs[32g + r - 32] otherwise) and the
 *   fifth bit is bit (2g + (r >= 32)) of qh[r mod 32]; q = nibble + 16 * bit.
 *   w_i = d * sc[j] * q_i - dmin * mn[j], j = i / 32.
 * Arithmetic and error codes as in q4k_oracle.h.
 */
#ifndef Q5K_ORACLE_H
#define Q5K_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_Q5K_BLOCK_BYTES = 176 };

/* 5-bit quant (0..31) of weight i (0..255) from the 32 high-bit bytes and the
 * 128 nibble bytes of a block. */
int oracle_q5k_quant(const uint8_t qh[32], const uint8_t qs[128], int i);

/* One 176-byte super-block -> 256 fp32 weights. */
void oracle_q5k_dequant_block(const uint8_t blk[176], float w[256]);

/* W [n, k] in Q5_K (n rows of k/256 blocks) -> fp32 [n, k] / bf16 bits [n, k]. */
int oracle_q5k_dequant_f32(const uint8_t *w, int64_t n, int64_t k, float *out);
int oracle_q5k_dequant_bf16(const uint8_t *w, int64_t n, int64_t k, uint16_t *out);

/* GEMV as oracle_gemv / oracle_gemv_rows, on Q5_K weights. */
int oracle_q5k_gemv(const uint8_t *w, const float *x, int64_t m, int64_t n,
                    int64_t k, double *y, double *a);
int oracle_q5k_gemv_rows(const uint8_t *w, const float *x, int64_t m, int64_t n,
                         int64_t k, const int64_t *rows, int64_t nrows,
                         double *y, double *a);

/* GEMM as oracle_gemm / oracle_gemm_cols (X bf16 bits [m, k]), on Q5_K weights. */
int oracle_q5k_gemm(const uint8_t *w, const uint16_t *x, int64_t m, int64_t n,
                    int64_t k, double *y, double *a);
int oracle_q5k_gemm_cols(const uint8_t *w, const uint16_t *x, int64_t m, int64_t n,
                         int64_t k, const int64_t *cols, int64_t ncols, double *y,
                         double *a);

#ifdef __cplusplus
}
#endif
#endif
