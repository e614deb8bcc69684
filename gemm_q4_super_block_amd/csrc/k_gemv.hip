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

#include <atomic>

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

// ---------------------------------------------------------------- batch 1
// x (up to kXChunk floats at a time) is staged once per workgroup in LDS,
// skewed by 16 bytes every 256 bytes so that the lanes of a wave -- whose
// 64-float slices start 256 bytes apart -- hit distinct banks; the staging
// pass also forms the 32-wide sub-block sums of x.  Each wave prefetches the
// next K step's weights before it computes the current one.
constexpr int kXChunk = 16384;

__device__ __forceinline__ int xs_index(int i) { return i + ((i >> 6) << 2); }

__host__ __device__ constexpr size_t gemv1_lds_bytes(int kc) {
  return static_cast<size_t>(kc + kc / 16 + kc / 32) * sizeof(float);
}

template <int R, bool GLU>
__global__ __launch_bounds__(256) void k_gemv1_q4k(const uint8_t* __restrict__ w,
                                                   const uint8_t* __restrict__ w2,
                                                   const float* __restrict__ x,
                                                   float* __restrict__ y, int n, int k) {
  constexpr int NW = GLU ? 2 : 1;
  extern __shared__ float smem[];
  const int kc_max = min(k, kXChunk);
  float* xs = smem;
  float* ssum = smem + kc_max + kc_max / 16;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int b = lane >> 2;
  const int g = lane & 3;
  const int kb_count = k >> 8;
  const int steps = (kb_count + 15) >> 4;
  const size_t row_bytes = static_cast<size_t>(kb_count) * kBlockBytes;
  const int row0 = (blockIdx.x * 4 + wave) * R;

  auto load_w = [&](int s, uint4 (&hd)[NW][R], uint4 (&qa)[NW][R], uint4 (&qb)[NW][R]) {
    const int kb = min(s * 16 + b, kb_count - 1);
#pragma unroll
    for (int u = 0; u < NW; ++u) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = min(row0 + r, n - 1);
        const uint8_t* p = (u ? w2 : w) + row * row_bytes + static_cast<size_t>(kb) * kBlockBytes;
        hd[u][r] = load16(p);
        qa[u][r] = load16(p + 16 + 32 * g);
        qb[u][r] = load16(p + 32 + 32 * g);
      }
    }
  };

  uint4 hd[NW][R], qa[NW][R], qb[NW][R];
  load_w(0, hd, qa, qb);  // in flight while x is staged

  float acc[NW][R];
#pragma unroll
  for (int u = 0; u < NW; ++u)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[u][r] = 0.0f;

  for (int c0 = 0; c0 < k; c0 += kXChunk) {
    const int kc = min(kXChunk, k - c0);
    if (c0 > 0) __syncthreads();  // every wave is done with the previous chunk
    for (int i0 = 16 * t; i0 < kc; i0 += 16 * 256) {
      const f4_t* src = reinterpret_cast<const f4_t*>(x + c0 + i0);
      const f4_t v0 = src[0], v1 = src[1], v2 = src[2], v3 = src[3];
      f4_t* dst = reinterpret_cast<f4_t*>(xs + xs_index(i0));
      dst[0] = v0;
      dst[1] = v1;
      dst[2] = v2;
      dst[3] = v3;
      float s = ((v0.x + v0.y) + (v0.z + v0.w)) + ((v1.x + v1.y) + (v1.z + v1.w)) +
                ((v2.x + v2.y) + (v2.z + v2.w)) + ((v3.x + v3.y) + (v3.z + v3.w));
      s += dpp_mov<0xB1>(s);  // thread t ^ 1 holds the other 16 floats of the sub-block
      if ((t & 1) == 0) ssum[i0 >> 5] = s;
    }
    __syncthreads();

    const int s_begin = c0 >> 12;
    const int s_end = min(steps, (c0 + kc + 4095) >> 12);
    for (int s = s_begin; s < s_end; ++s) {
      uint4 nhd[NW][R], nqa[NW][R], nqb[NW][R];
      const bool more = s + 1 < steps;
      if (more) load_w(s + 1, nhd, nqa, nqb);
      const bool active = s * 16 + b < kb_count;
      const int kb_local = active ? s * 16 + b - (c0 >> 8) : 0;
      const float* xb = xs + xs_index(kb_local * kQK + 64 * g);
      const float sl = active ? ssum[kb_local * 8 + 2 * g] : 0.0f;
      const float sh = active ? ssum[kb_local * 8 + 2 * g + 1] : 0.0f;
      float pl[NW][R], ph[NW][R];
#pragma unroll
      for (int u = 0; u < NW; ++u)
#pragma unroll
        for (int r = 0; r < R; ++r) pl[u][r] = ph[u][r] = 0.0f;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const f4_t xl = active ? *reinterpret_cast<const f4_t*>(xb + 4 * c) : f4_t{0, 0, 0, 0};
        const f4_t xh = active ? *reinterpret_cast<const f4_t*>(xb + 32 + 4 * c) : f4_t{0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < NW; ++u) {
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const uint32_t v = c < 4 ? word(qa[u][r], c) : word(qb[u][r], c - 4);
            const uint32_t lo = v & 0x0F0F0F0Fu;
            const uint32_t hi = (v >> 4) & 0x0F0F0F0Fu;
            const f2_t l01 = fp8x2_lo(lo), l23 = fp8x2_hi(lo);
            const f2_t h01 = fp8x2_lo(hi), h23 = fp8x2_hi(hi);
            float a = pl[u][r];
            a = __builtin_fmaf(l01.x, xl.x, a);
            a = __builtin_fmaf(l01.y, xl.y, a);
            a = __builtin_fmaf(l23.x, xl.z, a);
            a = __builtin_fmaf(l23.y, xl.w, a);
            pl[u][r] = a;
            float e = ph[u][r];
            e = __builtin_fmaf(h01.x, xh.x, e);
            e = __builtin_fmaf(h01.y, xh.y, e);
            e = __builtin_fmaf(h23.x, xh.z, e);
            e = __builtin_fmaf(h23.y, xh.w, e);
            ph[u][r] = e;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < NW; ++u) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const GroupScales sc = group_scales(hd[u][r], g);
          float a = acc[u][r];
          a = __builtin_fmaf(sc.a_lo, pl[u][r], a);
          a = __builtin_fmaf(sc.a_hi, ph[u][r], a);
          a = __builtin_fmaf(-sc.b_lo, sl, a);
          a = __builtin_fmaf(-sc.b_hi, sh, a);
          acc[u][r] = a;
          hd[u][r] = nhd[u][r];
          qa[u][r] = nqa[u][r];
          qb[u][r] = nqb[u][r];
        }
      }
    }
  }

#pragma unroll
  for (int r = 0; r < R; ++r) {
    float v = wave_sum(acc[0][r]);
    if constexpr (GLU) v = silu(v) * wave_sum(acc[NW - 1][r]);
    if (lane == 0 && row0 + r < n) y[row0 + r] = v;
  }
}

template <int R, bool GLU>
hipError_t launch1(const uint8_t* w, const uint8_t* w2, const float* x, float* y, int n, int k,
                   hipStream_t stream) {
  const size_t lds = gemv1_lds_bytes(min(k, kXChunk));
  // LDS above 64 KiB needs an opt-in per kernel and device (set once per device).
  static std::atomic<uint64_t> attr_set{0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipGetLastError();
  const uint64_t bit = 1ull << (dev & 63);
  if (!(attr_set.load(std::memory_order_acquire) & bit)) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemv1_q4k<R, GLU>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(gemv1_lds_bytes(kXChunk)));
    if (e != hipSuccess) return e;
    attr_set.fetch_or(bit, std::memory_order_acq_rel);
  }
  const int grid = (n + 4 * R - 1) / (4 * R);
  hipLaunchKernelGGL((k_gemv1_q4k<R, GLU>), dim3(grid), dim3(256), lds, stream, w, w2, x, y, n, k);
  return hipGetLastError();
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
      e = launch1<kGemvRowsPerWave, false>(w, w, xs, ys, (int)n, (int)k, stream);
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
  return launch1<kGateUpRowsPerWave, true>(w_gate, w_up, x, h, (int)d_ff, (int)d_model, stream);
}

}  // namespace q4k
