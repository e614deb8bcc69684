/*
 * q3k_oracle.h -- plain, slow CPU oracle for the Q3_K sibling format.
 *
 * TEST INFRASTRUCTURE ONLY, like q4k_oracle.h: only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it; it shares no code
 * with the HIP library.
 *
 * Source: "CPU kernel parity: decode and tile kernels at llama.cpp speed ..."
 * (daScript PR page), section on the kernel work: the 3-bit k-quant ("k3")
 * keeps its high bits in a plane (hmask) and flushes one scale per sub-block
 * into the accumulator, like k6.  The pages print no Q3_K layout; the reading
 * used here is the GGUF convention:
 *   110 bytes per 256 weights = hmask[32] at 0, qs[64] at 32, 12 scale bytes
 *   s[12] at 96, fp16 d (little-endian) at 108.
 *   Weight i = 128 h + 32 j + l (h = 0..1, j = 0..3, l = 0..31):
 *     low  = bits 2j, 2j+1 of qs[32 h + l];
 *     high = bit 4h + j of hmask[l];
 *     q    = low - 4 (1 - high), in -4..3.
 *   Sub-block t = i / 16 (0..15) has a 6-bit scale u_t: its low 4 bits are
 *   the low nibble of s[t] for t < 8 and the high nibble of s[t - 8] for
 *   t >= 8; its top 2 bits are bits 2 (t / 4), 2 (t / 4) + 1 of s[8 + t mod 4].
 *   sc_t = u_t - 32 (-32..31).
 *   w_i = d * sc_t * q_i, exact (at most 11 + 6 + 3 bits), rounded to fp32.
 * A matrix W [n, k] (k a multiple of 256) is n rows of k/256 consecutive
 * blocks.  Arithmetic and error codes as in q4k_oracle.h.
 */
#ifndef Q3K_ORACLE_H
#define Q3K_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_Q3K_BLOCK_BYTES = 110 };

/* Signed 3-bit quant (-4..3) of weight i (0..255) of a block. */
int oracle_q3k_quant(const uint8_t blk[110], int i);

/* Signed sub-block scale sc_t (-32..31), t = 0..15. */
int oracle_q3k_scale(const uint8_t blk[110], int t);

/* One 110-byte block -> 256 fp32 weights. */
void oracle_q3k_dequant_block(const uint8_t blk[110], float w[256]);

/* W [n, k] in Q3_K -> fp32 [n, k] / bf16 bits [n, k]. */
int oracle_q3k_dequant_f32(const uint8_t *w, int64_t n, int64_t k, float *out);
int oracle_q3k_dequant_bf16(const uint8_t *w, int64_t n, int64_t k, uint16_t *out);

/* GEMV as oracle_gemv / oracle_gemv_rows, on Q3_K weights. */
int oracle_q3k_gemv(const uint8_t *w, const float *x, int64_t m, int64_t n,
                    int64_t k, double *y, double *a);
int oracle_q3k_gemv_rows(const uint8_t *w, const float *x, int64_t m, int64_t n,
                         int64_t k, const int64_t *rows, int64_t nrows,
                         double *y, double *a);

/* GEMM as oracle_gemm / oracle_gemm_cols (X bf16 bits [m, k], Y = X W^T), on
 * Q3_K weights: the tile kernel's result ("CPU kernel parity ...":
 * each k-quant has a decode kernel and a tile kernel), from the fp32 weights
 * and the exactly decoded bf16 X, products summed in k order in fp64;
 * a = sum |X W| with the fp32 weights. */
int oracle_q3k_gemm(const uint8_t *w, const uint16_t *x, int64_t m, int64_t n,
                    int64_t k, double *y, double *a);
int oracle_q3k_gemm_cols(const uint8_t *w, const uint16_t *x, int64_t m, int64_t n,
                         int64_t k, const int64_t *cols, int64_t ncols,
                         double *y, double *a);

#ifdef __cplusplus
}
#endif
#endif
