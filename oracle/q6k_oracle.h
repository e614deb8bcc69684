/*
 * q6k_oracle.h -- plain, slow CPU oracle for the Q6_K sibling format.
 *
 * TEST INFRASTRUCTURE ONLY, like q4k_oracle.h: only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it; it shares no code
 * with the HIP library.
 *
 * Source: "CPU kernel parity: decode and tile kernels at llama.cpp speed ..."
 * (daScript PR page), section on the kernel work: the 6-bit k-quant ("k6")
 * keeps its two high bits in a plane beside the nibbles and flushes one
 * scale per sub-block into the accumulator.  The pages print no Q6_K layout;
 * the reading used here is the GGUF convention:
 *   210 bytes per 256 weights = ql[128] (low nibbles) at 0, qh[64] (high
 *   bit pairs) at 128, sc[16] (signed 8-bit sub-block scales) at 192, fp16 d
 *   (little-endian) at 208.
 *   Weight i = 128 h + 32 j + l (h = 0..1, j = 0..3, l = 0..31):
 *     nibble = ql[64 h + 32 (j mod 2) + l], low half for j < 2, high half
 *              for j >= 2;
 *     high   = bits 2j, 2j+1 of qh[32 h + l];
 *     q      = nibble + 16 high (0..63);
 *     w_i    = d * sc[i / 16] * (q - 32), the exact value rounded once to
 *              fp32 (|d sc (q - 32)| needs at most 11 + 7 + 6 bits).
 * A matrix W [n, k] (k a multiple of 256) is n rows of k/256 consecutive
 * blocks.  Arithmetic and error codes as in q4k_oracle.h.
 */
#ifndef Q6K_ORACLE_H
#define Q6K_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_Q6K_BLOCK_BYTES = 210 };

/* 6-bit quant (0..63) of weight i (0..255) of a block. */
int oracle_q6k_quant(const uint8_t blk[210], int i);

/* One 210-byte block -> 256 fp32 weights. */
void oracle_q6k_dequant_block(const uint8_t blk[210], float w[256]);

/* W [n, k] in Q6_K -> fp32 [n, k] / bf16 bits [n, k]. */
int oracle_q6k_dequant_f32(const uint8_t *w, int64_t n, int64_t k, float *out);
int oracle_q6k_dequant_bf16(const uint8_t *w, int64_t n, int64_t k, uint16_t *out);

/* GEMV as oracle_gemv / oracle_gemv_rows, on Q6_K weights. */
int oracle_q6k_gemv(const uint8_t *w, const float *x, int64_t m, int64_t n,
                    int64_t k, double *y, double *a);
int oracle_q6k_gemv_rows(const uint8_t *w, const float *x, int64_t m, int64_t n,
                         int64_t k, const int64_t *rows, int64_t nrows,
                         double *y, double *a);

/* GEMM as oracle_gemm / oracle_gemm_cols (X bf16 bits [m, k], Y = X W^T), on
 * Q6_K weights: the tile kernel's result ("CPU kernel parity ...":
 * each k-quant has a decode kernel and a tile kernel), from the fp32 weights
 * and the exactly decoded bf16 X, products summed in k order in fp64;
 * a = sum |X W| with the fp32 weights. */
int oracle_q6k_gemm(const uint8_t *w, const uint16_t *x, int64_t m, int64_t n,
                    int64_t k, double *y, double *a);
int oracle_q6k_gemm_cols(const uint8_t *w, const uint16_t *x, int64_t m, int64_t n,
                         int64_t k, const int64_t *cols, int64_t ncols,
                         double *y, double *a);

#ifdef __cplusplus
}
#endif
#endif
