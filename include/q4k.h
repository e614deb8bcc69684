/*
 * q4k.h -- C ABI of libq4k: the linear layer of LLM inference computed
 * directly on Q4_K block-quantized weights, on AMD Instinct MI355X (gfx950).
 *
 * Sources for what is computed, by page title and section:
 *   [P1] "Writing an ESIMD Fused Kernel From Reverse-Engineered Assembly":
 *        "Getting Q4_K Right" (Q4_K dequantization fused into a dot product),
 *        "Building ESIMD Infrastructure" (the MUL_MAT + MUL_MAT + SWIGLU MLP
 *        fusion), "SLM-Tiled GEMM and Graph Recording" (a shared-memory tiled
 *        GEMM for the prefill shape).
 *   [P2] "xpu-kernels -- fused kernels for Intel Arc (Xe2) ...": "Use from C"
 *        and "API" (int status codes, a last-error string, an init call,
 *        int64 sizes, entry points that enqueue on the caller's stream).
 *   [P3] "CPU kernel parity: decode and tile kernels at llama.cpp speed ..."
 *        (daScript PR page): the decode (GEMV) and tile (prefill) kernel
 *        split; "Validation" (every kernel bit-exact against the reference
 *        decode).
 *
 * Q4_K super-block (the pages name it and its 6-bit sub-block scales and
 * mins but print no byte layout; this is the layout the library reads):
 *   144 bytes encode 256 weights = 8 sub-blocks of 32.
 *     bytes 0..1    d     fp16, little-endian: multiplies the 6-bit scales
 *     bytes 2..3    dmin  fp16, little-endian: multiplies the 6-bit mins
 *     bytes 4..15   s[12] eight 6-bit scales sc[0..7] and eight 6-bit mins
 *                   mn[0..7]: for j < 4, sc[j] = s[j] & 63, mn[j] =
 *                   s[j+4] & 63; for j >= 4, sc[j] = (s[j+4] & 15) |
 *                   (s[j-4] >> 6) << 4 and mn[j] = (s[j+4] >> 4) |
 *                   (s[j] >> 6) << 4
 *     bytes 16..143 qs[128] 4-bit quants: in group g = 0..3, the low nibble
 *                   of qs[32g + r] is weight 64g + r and its high nibble is
 *                   weight 64g + 32 + r (r = 0..31)
 *   weight i = d * sc[i/32] * q_i - dmin * mn[i/32], rounded once to fp32.
 * A matrix W [n, k] (k a multiple of 256) is n rows of k/256 consecutive
 * super-blocks, row-major: block b of row r starts at byte (r*k/256 + b)*144.
 *
 * Conventions for every entry point:
 *   - Pointers are device pointers on the current HIP device (memory from
 *     hipMalloc or torch's CUDA allocator); the caller owns all memory.  The
 *     library allocates, frees and synchronizes nothing on these calls.
 *   - Calls enqueue asynchronously on `stream` (a hipStream_t; NULL = the
 *     null stream) and return once the work is enqueued.
 *   - Sizes are int64; byte offsets are computed in 64 bits.
 *   - Arguments are validated before anything touches the device; on a
 *     non-zero return nothing was enqueued and q4k_last_error() holds the
 *     reason (thread-local, valid until this thread's next call).
 *   - Outputs must not overlap inputs.
 */
#ifndef LIBQ4K_Q4K_H
#define LIBQ4K_Q4K_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define Q4K_OK 0
#define Q4K_ERR_INVALID_ARG (-1) /* null pointer, size out of range, k % 256 */
#define Q4K_ERR_ALIGN (-2)       /* a pointer is not 16-byte aligned */
#define Q4K_ERR_DEVICE (-3)      /* no HIP device, or it is not gfx950 */
#define Q4K_ERR_LAUNCH (-4)      /* the HIP runtime rejected a launch */

/* Weights per super-block, bytes per super-block, largest GEMV batch. */
#define Q4K_QK 256
#define Q4K_BLOCK_BYTES 144
#define Q4K_GEMV_MAX_M 32
/* Largest n (weight rows) of any GEMV or GEMM: tile indices stay in int32. */
#define Q4K_MAX_N 2147418111 /* 2^31 - 1 - 65536 */
/* Largest k of the GEMMs (q4k_, q5k_, q6k_, q3k_gemm): a 256-row weight tile
 * spans less than 4 GiB, so in-tile byte offsets fit 32 bits; the tile's base
 * and every other offset are 64-bit.  Matrices of any total size (above
 * 4 GiB included) are addressed correctly. */
#define Q4K_GEMM_MAX_K 16777216
/* Bytes per Q5_K super-block (the q5k_ entry points). */
#define Q5K_BLOCK_BYTES 176
/* Bytes per Q6_K block (the q6k_ entry points). */
#define Q6K_BLOCK_BYTES 210
/* Bytes per Q3_K block (the q3k_ entry points). */
#define Q3K_BLOCK_BYTES 110

/* Checks that a HIP device is present and is gfx950, for the current device.
 * Idempotent and cheap after the first call per device; the compute entry
 * points call it themselves.  Returns Q4K_OK or Q4K_ERR_DEVICE. [P2 "API":
 * an explicit init call.] */
int q4k_init(void);

/* gcnArchName of the current device ("gfx950:sramecc+:xnack-" or similar),
 * or "none".  The string is owned by the library. [P2 "API".] */
const char* q4k_device_name(void);

/* Message for the last non-zero return on the calling thread ("" if none).
 * Owned by the library. [P2 "API": a last-error string.] */
const char* q4k_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int q4k_version(void);

/* Decode GEMV at batch m (decode step, or a small batch of tokens).
 *   y[i, j] = sum_c W[j, c] * x[i, c]   for i < m, j < n, c < k.
 *   w: Q4_K matrix [n, k] (layout above), 16-byte aligned.
 *   x: fp32 [m, k] row-major, 16-byte aligned.
 *   y: fp32 [m, n] row-major, 16-byte aligned.
 *   1 <= m <= Q4K_GEMV_MAX_M, n >= 1, k >= 256 with k % 256 == 0.
 * Each weight is formed exactly (the dequant export's fp32 value) before it
 * meets x: for m <= 4 in an fp32 FMA dot product, for 5 <= m <= 32 on bf16
 * MFMA with weight and x each split into bf16 hi + lo parts.  Each output
 * lies within 1e-4 * sum_c |W[j,c] x[i,c]| of the exact value, and is +-0
 * when every product W[j,c] x[i,c] is zero.
 * [P1 "Getting Q4_K Right"; P3 decode kernels.] */
int q4k_gemv(const void* w, const float* x, float* y, int64_t m, int64_t n,
             int64_t k, void* stream);

/* Largest layer count and largest k of q4k_gemv_layers. */
#define Q4K_LAYERS_MAX 32
#define Q4K_LAYERS_MAX_K 16384

/* Several independent decode GEMVs of one shape in one launch.
 *   y[l][j] = sum_c W[l][j, c] * x[l][c]   for l < layers, j < n, c < k.
 *   w, x, y: host arrays of `layers` device pointers (read during the call;
 *   the caller keeps ownership): w[l] a Q4_K matrix [n, k], x[l] fp32 [k],
 *   y[l] fp32 [n], each 16-byte aligned.  Layers may share x (the Q, K and V
 *   projections of one token) or not (the experts a token routes to).
 *   1 <= layers <= Q4K_LAYERS_MAX, n >= 1, 256 <= k <= Q4K_LAYERS_MAX_K with
 *   k % 256 == 0.
 * Each y[l] is what q4k_gemv(w[l], x[l], y[l], 1, n, k) computes (the same
 * tolerance and the same per-row arithmetic).  Recording the work of a decode
 * step so that launch overhead is paid once is the lever of [P1 "SLM-Tiled
 * GEMM and Graph Recording"]; here one persistent dispatch streams every
 * layer's weights back to back, the next layer's rows in flight while the
 * current ones are computed.  No y[l] may overlap any w, x or other y.
 * Errors as for q4k_gemv, reported for the first layer that fails. */
int q4k_gemv_layers(const void* const* w, const float* const* x, float* const* y,
                    int64_t layers, int64_t n, int64_t k, void* stream);

/* Prefill GEMM.
 *   Y[i, j] = sum_c X[i, c] * W[j, c]   for i < m, j < n  (Y = X W^T).
 *   w: Q4_K matrix [n, k], 16-byte aligned.
 *   x_bf16: bf16 bit patterns [m, k] row-major, 16-byte aligned.
 *   y: fp32 [m, n] row-major, 16-byte aligned.
 *   m >= 1, n >= 1, k >= 256 with k % 256 == 0.
 * Weights are dequantized to bf16 (round to nearest even of the fp32 weight)
 * -- in registers or through LDS, by shape -- and contracted on bf16 MFMA
 * with fp32 accumulation; each output lies within 1e-2 * sum_c |W[j,c] X[i,c]|
 * of the exact value.
 * [P1 "SLM-Tiled GEMM and Graph Recording"; P3 tile kernels.] */
int q4k_gemm(const void* w, const uint16_t* x_bf16, float* y, int64_t m,
             int64_t n, int64_t k, void* stream);

/* SwiGLU MLP at one token (M = 1).
 *   h   = silu(W_gate x) * (W_up x),  silu(t) = t / (1 + exp(-t))
 *   out = W_down h
 *   w_gate, w_up: Q4_K [d_ff, d_model];  w_down: Q4_K [d_model, d_ff].
 *   x: fp32 [d_model];  h: fp32 [d_ff] (caller-owned scratch, left valid);
 *   out: fp32 [d_model].  All 16-byte aligned.
 *   d_model and d_ff: positive multiples of 256.
 * Gate and up share one read of x and h is formed in registers; the down
 * projection is a second launch on the same stream (it needs all of h).
 * [P1 "Building ESIMD Infrastructure": MUL_MAT + MUL_MAT + SWIGLU.] */
int q4k_swiglu_mlp(const void* w_gate, const void* w_up, const void* w_down,
                   const float* x, float* h, float* out, int64_t d_model,
                   int64_t d_ff, void* stream);

/* Largest d_ff of q4k_swiglu_mlp_noalloc (the size of its device scratch). */
#define Q4K_NOALLOC_MAX_D_FF 65536

/* The SwiGLU MLP for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * as q4k_swiglu_mlp, but h lives in the library's own scratch, a static
 * device array of Q4K_NOALLOC_MAX_D_FF floats (256 KiB) that each GPU the
 * library runs on holds until the process ends.  Nothing is allocated or
 * freed on any call; the scratch address is resolved once per device
 * (hipGetSymbolAddress) on the first call with that device current.
 *   out fp32 [d_model]; the other arguments as for q4k_swiglu_mlp;
 *   d_ff <= Q4K_NOALLOC_MAX_D_FF, else Q4K_ERR_INVALID_ARG.
 * Every call on one GPU shares that GPU's scratch: calls that overlap in time
 * on one GPU (different streams, or threads without ordering) race on h and
 * give wrong results; calls in one stream are ordered and safe.  h is written
 * in full before it is read, so nothing needs clearing between calls.
 * Errors as for q4k_swiglu_mlp, plus Q4K_ERR_DEVICE if the runtime cannot
 * give the scratch address. */
int q4k_swiglu_mlp_noalloc(const void* w_gate, const void* w_up, const void* w_down,
                           const float* x, float* out, int64_t d_model, int64_t d_ff,
                           void* stream);

/* Diagnostic dequantization of W [n, k] to fp32 / to bf16 bit patterns,
 * row-major [n, k], through the same device routine the GEMM fills LDS with.
 * The fp32 result is the exact weight rounded once to nearest even; the bf16
 * result is that fp32 value rounded to nearest even.  out 16-byte aligned.
 * [P3 "Validation": bit-exact against the reference decode.] */
int q4k_dequantize_f32(const void* w, float* out, int64_t n, int64_t k,
                       void* stream);
int q4k_dequantize_bf16(const void* w, uint16_t* out, int64_t n, int64_t k,
                        void* stream);

/* Measurement aid, not part of the method: streams `bytes` of buf with
 * 16-byte loads and discards them (sink, 4 bytes of device memory, is
 * written only on a 2^-32 coincidence of the data).  Timed on the same cold
 * buffers as a GEMV, it gives the read rate that working-set size allows.
 *   buf 16-byte aligned, bytes a positive multiple of 16; sink 4-byte aligned.
 * Errors: Q4K_ERR_INVALID_ARG, Q4K_ERR_ALIGN, Q4K_ERR_DEVICE, Q4K_ERR_LAUNCH. */
int q4k_read_probe(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

/* ---- Q5_K, the 5-bit sibling ------------------------------------------------
 * [P3, the kernel work: the 4-bit and 5-bit k-quants are decoded by the same
 * fused kernel shape.]
 * The pages print no Q5_K layout either; the library reads the Q4_K
 * super-block with one high-bit plane added:
 *   176 bytes encode 256 weights.
 *     bytes 0..15    d, dmin and s[12] exactly as in Q4_K
 *     bytes 16..47   qh[32]: bit (2g + [r >= 32]) of qh[r mod 32] is the fifth
 *                    bit of weight 64g + r
 *     bytes 48..175  qs[128]: the 4-bit nibbles, Q4_K's map
 *   q_i = nibble_i + 16 * bit_i (0..31); weight i = d * sc[i/32] * q_i -
 *   dmin * mn[i/32], rounded once to fp32.
 * A matrix is laid out as for Q4_K with 176-byte blocks. */

/* Decode GEMV on Q5_K weights: as q4k_gemv (same x, y, m, n, k, tolerance
 * and errors; the same two kernel families by m) with w a Q5_K matrix
 * [n, k], 16-byte aligned. */
int q5k_gemv(const void* w, const float* x, float* y, int64_t m, int64_t n,
             int64_t k, void* stream);

/* Prefill GEMM on Q5_K weights: as q4k_gemm (same x_bf16, y, m, n, k,
 * tolerance and errors) with w a Q5_K matrix [n, k].  Each step's weight tile
 * is dequantized to bf16 in LDS (the same rounding), with split K on small
 * grids. */
int q5k_gemm(const void* w, const uint16_t* x_bf16, float* y, int64_t m,
             int64_t n, int64_t k, void* stream);

/* Diagnostic dequantization of a Q5_K matrix: as q4k_dequantize_f32 / _bf16
 * (exact weight rounded once to fp32; bf16 = nearest even of that). */
int q5k_dequantize_f32(const void* w, float* out, int64_t n, int64_t k,
                       void* stream);
int q5k_dequantize_bf16(const void* w, uint16_t* out, int64_t n, int64_t k,
                        void* stream);

/* ---- Q6_K, the 6-bit sibling ------------------------------------------------
 * [P3, the kernel work: "k6" keeps its two high bits in a plane and flushes
 * one scale per sub-block into the accumulator.]  The pages print no Q6_K
 * layout; the library reads the GGUF one:
 *   210 bytes encode 256 weights = 16 sub-blocks of 16.
 *     bytes 0..127    ql[128]: weight 128h + 32j + l (h = 0..1, j = 0..3,
 *                     l = 0..31) has its low 4 bits in the low (j < 2) or
 *                     high (j >= 2) nibble of ql[64h + 32(j mod 2) + l]
 *     bytes 128..191  qh[64]: its top 2 bits are bits 2j, 2j+1 of qh[32h + l]
 *     bytes 192..207  sc[16]: signed 8-bit sub-block scales
 *     bytes 208..209  d, fp16, little-endian
 *   weight i = d * sc[i/16] * (q_i - 32), q_i = 0..63, rounded once to fp32.
 * A matrix is laid out as for Q4_K with 210-byte blocks (a block may start 2
 * bytes past a 4-byte boundary; the matrix itself must be 16-byte aligned). */

/* Decode GEMV on Q6_K weights: as q4k_gemv (same x, y, m, n, k, tolerance
 * and errors) with w a Q6_K matrix [n, k], 16-byte aligned.  A batch (m > 1)
 * streams W once per 4 x rows.  Each sub-block's scale multiplies a sum of
 * exact (q - 32) x products, so a zero weight adds exactly zero. */
int q6k_gemv(const void* w, const float* x, float* y, int64_t m, int64_t n,
             int64_t k, void* stream);

/* Prefill GEMM on Q6_K weights: as q4k_gemm (same x_bf16, y, m, n, k,
 * tolerance and errors) with w a Q6_K matrix [n, k], 16-byte aligned.  Each
 * step's weight tile is dequantized to bf16 in LDS (the exact weight rounded
 * to fp32, then to bf16), with split K on small grids. */
int q6k_gemm(const void* w, const uint16_t* x_bf16, float* y, int64_t m,
             int64_t n, int64_t k, void* stream);

/* Diagnostic dequantization of a Q6_K matrix: as q4k_dequantize_f32 / _bf16
 * (exact weight rounded once to fp32; bf16 = nearest even of that). */
int q6k_dequantize_f32(const void* w, float* out, int64_t n, int64_t k,
                       void* stream);
int q6k_dequantize_bf16(const void* w, uint16_t* out, int64_t n, int64_t k,
                        void* stream);

/* ---- Q3_K, the 3-bit sibling ------------------------------------------------
 * [P3, the kernel work: "k3", like k6, keeps its high bits in a plane and
 * flushes one scale per sub-block into the accumulator.]  The pages print no
 * Q3_K layout; the library reads the GGUF one:
 *   110 bytes encode 256 weights = 16 sub-blocks of 16.
 *     bytes 0..31     hmask[32]: the third bit of weight 128h + 32j + l is bit
 *                     4h + j of hmask[l]
 *     bytes 32..95    qs[64]: its low two bits are bits 2j, 2j+1 of qs[32h + l]
 *     bytes 96..107   s[12]: sub-block t's 6-bit scale u_t has the low nibble
 *                     of s[t] (t < 8) or the high nibble of s[t - 8], and bits
 *                     2(t/4), 2(t/4)+1 of s[8 + t mod 4] on top
 *     bytes 108..109  d, fp16, little-endian
 *   weight i = d * (u_{i/16} - 32) * (q_i - 4), q_i = 0..7 (exact in fp32).
 * A matrix is laid out as for Q4_K with 110-byte blocks (16-byte aligned). */

/* Decode GEMV on Q3_K weights: as q4k_gemv (same x, y, m, n, k, tolerance
 * and errors) with w a Q3_K matrix [n, k], 16-byte aligned.  A batch (m > 1)
 * streams W once per 4 x rows.  Each sub-block's scale multiplies a sum of
 * exact (q - 4) x products, so a zero weight adds exactly zero. */
int q3k_gemv(const void* w, const float* x, float* y, int64_t m, int64_t n,
             int64_t k, void* stream);

/* Prefill GEMM on Q3_K weights: as q6k_gemm with w a Q3_K matrix [n, k]. */
int q3k_gemm(const void* w, const uint16_t* x_bf16, float* y, int64_t m,
             int64_t n, int64_t k, void* stream);

/* Diagnostic dequantization of a Q3_K matrix (the exact weight in fp32; bf16 =
 * nearest even of that). */
int q3k_dequantize_f32(const void* w, float* out, int64_t n, int64_t k,
                       void* stream);
int q3k_dequantize_bf16(const void* w, uint16_t* out, int64_t n, int64_t k,
                        void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LIBQ4K_Q4K_H */
