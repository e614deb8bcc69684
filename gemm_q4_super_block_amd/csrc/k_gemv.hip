// k_gemv.hip -- decode GEMV on Q4_K weights, and the gate/up SwiGLU stage.
//
// y[i, r] = sum_c W[r, c] x[i, c] for a few activation rows i (decode: one).
// The dequantization is fused into an fp32 FMA dot product ("Writing an
// ESIMD Fused Kernel From Reverse-Engineered Assembly", "Getting Q4_K Right":
// dequant feeding a dot with a SIMD reduce), and the gate and up projections
// of the MLP share one read of x with h = silu(g) * u formed in registers
// ("Building ESIMD Infrastructure": MUL_MAT + MUL_MAT + SWIGLU).
//
// Work mapping (wave64, 4 waves per workgroup):
//   * lane = 4*b + g: b = 0..15 is a super-block slot, g = 0..3 a quant group.
//     One step of the K loop covers 16 consecutive super-blocks of a row
//     (4096 weights); a lane reads the block header (16 B) and the 32 quant
//     bytes of its group (two 16-byte loads) -- weights 64g..64g+63 of the
//     block: 32 low nibbles of sub-block 2g and 32 high nibbles of 2g+1.
//   * a wave owns R consecutive weight rows (2R with the gate/up pair) and
//     reuses each x value it loads for all of them.
//   * per sub-block j the dot is refactored as
//       sum_l (a_j q_l - b_j) x_l = a_j * sum_l q_l x_l - b_j * sum_l x_l,
//     so the scales are applied twice per 32 weights, not per weight.
//   * quants are widened with v_cvt_pk_f32_fp8 (a masked nibble byte is the
//     fp8 value q * 2^-9), two per instruction.
//   * lanes reduce with DPP and two cross-row swizzles; lane 0 stores.
#include <hip/hip_runtime.h>

#include "q4k_device.h"
#include "q4k_launch.h"

namespace q4k {
namespace {

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

__device__ __forceinline__ float silu(float t) { return t / (1.0f + expf(-t)); }

template <int MT>
constexpr int kChunkUnroll = MT == 1 ? 2 : 1;

template <int MT, int R, bool GLU>
__global__ __launch_bounds__(256) void k_gemv_q4k(const uint8_t* __restrict__ w,
                                                  const uint8_t* __restrict__ w2,
                                                  const float* __restrict__ x,
                                                  float* __restrict__ y, int m, int n, int k) {
  constexpr int NW = GLU ? 2 : 1;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int b = lane >> 2;
  const int g = lane & 3;
  const int kb_count = k >> 8;
  const int row0 = (blockIdx.x * 4 + wave) * R;
  if (row0 >= n) return;  // whole wave idle; the kernel has no barriers
  const size_t row_bytes = static_cast<size_t>(kb_count) * kBlockBytes;

  float acc[NW][R][MT];
#pragma unroll
  for (int t = 0; t < NW; ++t)
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int i = 0; i < MT; ++i) acc[t][r][i] = 0.0f;

  for (int kb0 = 0; kb0 < kb_count; kb0 += 16) {
    const bool active = kb0 + b < kb_count;
    // Inactive lanes (ragged last step) read a valid block and see x = 0.
    const int kb = active ? kb0 + b : kb_count - 1;

    uint4 hd[NW][R], qa[NW][R], qb[NW][R];
#pragma unroll
    for (int t = 0; t < NW; ++t) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = min(row0 + r, n - 1);
        const uint8_t* p = (t ? w2 : w) + row * row_bytes + static_cast<size_t>(kb) * kBlockBytes;
        hd[t][r] = load16(p);
        qa[t][r] = load16(p + 16 + 32 * g);
        qb[t][r] = load16(p + 32 + 32 * g);
      }
    }

    float pl[NW][R][MT], ph[NW][R][MT], sl[MT], sh[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      sl[i] = 0.0f;
      sh[i] = 0.0f;
#pragma unroll
      for (int t = 0; t < NW; ++t)
#pragma unroll
        for (int r = 0; r < R; ++r) pl[t][r][i] = ph[t][r][i] = 0.0f;
    }

    const float* xb = x + static_cast<size_t>(kb) * kQK + 64 * g;
    // Two 16-byte quant chunks per lane; batched variants keep one chunk's x
    // live at a time (a rolled loop), batch 1 unrolls both for load depth.
#pragma unroll(kChunkUnroll<MT>)
    for (int hq = 0; hq < 2; ++hq) {
      uint4 qv[NW][R];
#pragma unroll
      for (int t = 0; t < NW; ++t)
#pragma unroll
        for (int r = 0; r < R; ++r) qv[t][r] = hq ? qb[t][r] : qa[t][r];
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const int c = 4 * hq + c4;
        f4_t xl[MT], xh[MT];
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          if (active && i < m) {
            xl[i] = *reinterpret_cast<const f4_t*>(xb + static_cast<size_t>(i) * k + 4 * c);
            xh[i] = *reinterpret_cast<const f4_t*>(xb + static_cast<size_t>(i) * k + 32 + 4 * c);
          } else {
            xl[i] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
            xh[i] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
          }
          sl[i] += (xl[i].x + xl[i].y) + (xl[i].z + xl[i].w);
          sh[i] += (xh[i].x + xh[i].y) + (xh[i].z + xh[i].w);
        }
#pragma unroll
        for (int t = 0; t < NW; ++t) {
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const uint32_t v = word(qv[t][r], c4);
            const uint32_t lo = v & 0x0F0F0F0Fu;
            const uint32_t hi = (v >> 4) & 0x0F0F0F0Fu;
            const f2_t l01 = fp8x2_lo(lo), l23 = fp8x2_hi(lo);
            const f2_t h01 = fp8x2_lo(hi), h23 = fp8x2_hi(hi);
#pragma unroll
            for (int i = 0; i < MT; ++i) {
              float a = pl[t][r][i];
              a = __builtin_fmaf(l01.x, xl[i].x, a);
              a = __builtin_fmaf(l01.y, xl[i].y, a);
              a = __builtin_fmaf(l23.x, xl[i].z, a);
              a = __builtin_fmaf(l23.y, xl[i].w, a);
              pl[t][r][i] = a;
              float e = ph[t][r][i];
              e = __builtin_fmaf(h01.x, xh[i].x, e);
              e = __builtin_fmaf(h01.y, xh[i].y, e);
              e = __builtin_fmaf(h23.x, xh[i].z, e);
              e = __builtin_fmaf(h23.y, xh[i].w, e);
              ph[t][r][i] = e;
            }
          }
        }
      }
    }

#pragma unroll
    for (int t = 0; t < NW; ++t) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const GroupScales s = group_scales(hd[t][r], g);
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          float a = acc[t][r][i];
          a = __builtin_fmaf(s.a_lo, pl[t][r][i], a);
          a = __builtin_fmaf(s.a_hi, ph[t][r][i], a);
          a = __builtin_fmaf(-s.b_lo, sl[i], a);
          a = __builtin_fmaf(-s.b_hi, sh[i], a);
          acc[t][r][i] = a;
        }
      }
    }
  }

#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int row = row0 + r;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      float v = wave_sum(acc[0][r][i]);
      if constexpr (GLU) {
        const float u = wave_sum(acc[NW - 1][r][i]);
        v = silu(v) * u;
      }
      if (lane == 0 && row < n && i < m) y[static_cast<size_t>(i) * n + row] = v;
    }
  }
}

template <int MT, int R, bool GLU>
hipError_t launch(const uint8_t* w, const uint8_t* w2, const float* x, float* y, int m, int n,
                  int k, hipStream_t stream) {
  const int rows_per_block = 4 * R;
  const int grid = (n + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL((k_gemv_q4k<MT, R, GLU>), dim3(grid), dim3(256), 0, stream, w, w2, x, y, m,
                     n, k);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const uint8_t* w, const float* x, float* y, int64_t m, int64_t n,
                       int64_t k, hipStream_t stream) {
  // Batches above 8 rows run as passes of 8 over x and y; W is re-streamed.
  for (int64_t i0 = 0; i0 < m; i0 += 8) {
    const int mm = static_cast<int>(m - i0 < 8 ? m - i0 : 8);
    const float* xs = x + i0 * k;
    float* ys = y + i0 * n;
    hipError_t e;
    if (mm == 1) {
      e = launch<1, kGemvRowsPerWave, false>(w, w, xs, ys, 1, (int)n, (int)k, stream);
    } else if (mm == 2) {
      e = launch<2, 2, false>(w, w, xs, ys, mm, (int)n, (int)k, stream);
    } else if (mm <= 4) {
      e = launch<4, 2, false>(w, w, xs, ys, mm, (int)n, (int)k, stream);
    } else {
      e = launch<8, 1, false>(w, w, xs, ys, mm, (int)n, (int)k, stream);
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_gateup_swiglu(const uint8_t* w_gate, const uint8_t* w_up, const float* x,
                                float* h, int64_t d_model, int64_t d_ff, hipStream_t stream) {
  return launch<1, kGateUpRowsPerWave, true>(w_gate, w_up, x, h, 1, (int)d_ff, (int)d_model,
                                             stream);
}

}  // namespace q4k
