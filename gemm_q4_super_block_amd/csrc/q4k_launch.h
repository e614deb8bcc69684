// q4k_launch.h -- host-side launchers of the libq4k kernels (internal).
//
// Each launcher enqueues on `stream` and returns the HIP status of the
// launch.  Arguments are validated by the C ABI (q4k_api.hip) beforehand:
// k % 256 == 0, sizes fit in int32, pointers 16-byte aligned.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4k {

// Shipped launch shapes (pinned by tests/test_abi.py).
constexpr int kGemvRowsPerWave = 1;    // decode GEMV, batch 1: rows of W per wave
constexpr int kGateUpRowsPerWave = 1;  // gate/up SwiGLU: row pairs per wave
// Prefill GEMMs with M >= 256 and at least this many 128 x 256 output tiles
// use the large-tile kernel.
constexpr int kGemmBigTiles = 128;
// Other prefill GEMMs (M > 32) with at least this many 64 x 128 output tiles
// use the mid-tile kernel; smaller grids split K over 128 x 128 tiles.
constexpr int kGemmMidTiles = 192;
// Batches of at most 32 rows with at least this many 64-row weight tiles use
// the streaming kernel; smaller ones split K over 128-row tiles.
constexpr int kGemmSmallTiles = 128;
// Batch-1 GEMVs outside the decode kernel with at most this many rows run 16
// waves per workgroup.
constexpr int64_t kGemvWideRows = 8192;
// Waves (rows) per workgroup of the batch-1 decode kernel (Q4_K, k <= 16384).
constexpr int kDecodeWaves = 8;
// Waves per workgroup of the MLP's gate/up decode kernel (a gate and an up
// wave per row) for d_model <= 16384.
constexpr int kDecodeGluWaves = 8;
// Q4_K and Q5_K GEMV batches of at least this many rows (up to 32) take the
// split-bf16 MFMA kernel (k_gemv_split.hip) instead of the fp32 FMA passes
// (which handle 1 to kGemvSplitMinM - 1 rows in one pass).
constexpr int kGemvSplitMinM = 5;

hipError_t launch_gemv(const uint8_t* w, const float* x, float* y, int64_t m, int64_t n,
                       int64_t k, hipStream_t stream);

// Independent batch-1 GEMVs of one shape in one launch (1 <= layers <= kGemvMaxLayers,
// k <= kGemvLayersMaxK): y[l] = W[l] x[l]; w, x, y are host arrays of device pointers.
constexpr int kGemvMaxLayers = 32;
constexpr int kGemvLayersMaxK = 16384;
hipError_t launch_gemv_layers(const uint8_t* const* w, const float* const* x, float* const* y,
                              int64_t layers, int64_t n, int64_t k, hipStream_t stream);

// Split-bf16 MFMA GEMV for kGemvSplitMinM <= m <= 32 (Q4_K, Q5_K).
bool gemv_split_supported(int64_t m);
hipError_t launch_gemv_split(const uint8_t* w, const float* x, float* y, int64_t m, int64_t n,
                             int64_t k, hipStream_t stream);
hipError_t launch_q5k_gemv_split(const uint8_t* w, const float* x, float* y, int64_t m, int64_t n,
                                 int64_t k, hipStream_t stream);

hipError_t launch_gateup_swiglu(const uint8_t* w_gate, const uint8_t* w_up, const float* x,
                                float* h, int64_t d_model, int64_t d_ff, hipStream_t stream);

hipError_t launch_dequant_f32(const uint8_t* w, float* out, int64_t n, int64_t k,
                              hipStream_t stream);
hipError_t launch_dequant_bf16(const uint8_t* w, uint16_t* out, int64_t n, int64_t k,
                               hipStream_t stream);

// Q5_K (176-byte super-blocks): GEMV and the dequant exports.
hipError_t launch_q5k_gemv(const uint8_t* w, const float* x, float* y, int64_t m, int64_t n,
                           int64_t k, hipStream_t stream);
hipError_t launch_q5k_gemm(const uint8_t* w, const uint16_t* x, float* y, int64_t m, int64_t n,
                           int64_t k, hipStream_t stream);
hipError_t launch_q5k_dequant_f32(const uint8_t* w, float* out, int64_t n, int64_t k,
                                  hipStream_t stream);
hipError_t launch_q5k_dequant_bf16(const uint8_t* w, uint16_t* out, int64_t n, int64_t k,
                                   hipStream_t stream);

hipError_t launch_gemm(const uint8_t* w, const uint16_t* x, float* y, int64_t m, int64_t n,
                       int64_t k, hipStream_t stream);
// Q4_K and Q5_K GEMM for m <= 32 (k_gemm_stream.hip); gemm_stream_tiles(n)
// counts its 64-row weight tiles.
int gemm_stream_tiles(int64_t n);
hipError_t launch_gemm_stream(const uint8_t* w, const uint16_t* x, float* y, int64_t m, int64_t n,
                              int64_t k, hipStream_t stream);
hipError_t launch_q5k_gemm_stream(const uint8_t* w, const uint16_t* x, float* y, int64_t m,
                                  int64_t n, int64_t k, hipStream_t stream);

// Q6_K (210-byte blocks): GEMV (passes of up to 4 x rows) and the dequant exports.
hipError_t launch_q6k_gemv(const uint8_t* w, const float* x, float* y, int64_t m, int64_t n,
                           int64_t k, hipStream_t stream);
hipError_t launch_q6k_dequant_f32(const uint8_t* w, float* out, int64_t n, int64_t k,
                                  hipStream_t stream);
hipError_t launch_q6k_dequant_bf16(const uint8_t* w, uint16_t* out, int64_t n, int64_t k,
                                   hipStream_t stream);

// Prefill GEMMs on the plane formats (X bf16 [m, k], fp32 Y).
hipError_t launch_q6k_gemm(const uint8_t* w, const uint16_t* x, float* y, int64_t m, int64_t n,
                           int64_t k, hipStream_t stream);
hipError_t launch_q3k_gemm(const uint8_t* w, const uint16_t* x, float* y, int64_t m, int64_t n,
                           int64_t k, hipStream_t stream);

// Q3_K (110-byte blocks): GEMV (passes of up to 4 x rows) and the dequant exports.
hipError_t launch_q3k_gemv(const uint8_t* w, const float* x, float* y, int64_t m, int64_t n,
                           int64_t k, hipStream_t stream);
hipError_t launch_q3k_dequant_f32(const uint8_t* w, float* out, int64_t n, int64_t k,
                                  hipStream_t stream);
hipError_t launch_q3k_dequant_bf16(const uint8_t* w, uint16_t* out, int64_t n, int64_t k,
                                   hipStream_t stream);

// INT8 W8A8 linear layer (k % 128 == 0, pointers 16-byte aligned).
hipError_t launch_w8a8_linear(const int8_t* x, const float* x_scale, const int8_t* w,
                              const float* w_scale, const float* bias, uint16_t* out, int64_t m,
                              int64_t n, int64_t k, hipStream_t stream);
hipError_t launch_w8a8_linear_acc(const int8_t* x, const int8_t* w, int32_t* acc, int64_t m,
                                  int64_t n, int64_t k, hipStream_t stream);
hipError_t launch_w8a8_epilogue(const int32_t* acc, uint16_t* out, const float* x_scale,
                                const float* w_scale, const float* bias, int64_t m, int64_t n,
                                hipStream_t stream);
hipError_t launch_w8a8_quantize_rows(const uint16_t* x, int8_t* q, float* scale, int64_t rows,
                                     int64_t k, hipStream_t stream);

hipError_t launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink,
                             hipStream_t stream);

}  // namespace q4k
