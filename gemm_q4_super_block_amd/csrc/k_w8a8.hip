// k_w8a8.hip -- INT8 W8A8 linear layer: int8 x int8 -> int32 on int8 MFMA,
// the dequant epilogue fused, plus the standalone epilogue and the row
// quantizer.
//
// What is computed ("xpu-kernels -- fused kernels for Intel Arc (Xe2) ...",
// sections "API", "Use from C" and "Quick start"): activations int8 [m, k]
// with one fp32 scale per row, weights int8 [n, k] with one fp32 scale per
// row (per output column of y = x w^T), acc[m, n] = sum_k x w exactly in
// int32, and out = bf16(acc * x_scale[m] * w_scale[n] + bias[n]).  The fp32
// operations are rounded one by one, left to right, none fused; the fused and
// the unfused paths therefore give identical bits.
//
// GEMM design for gfx950:
//   * workgroup = 4 waves as 2 x 2 over a (64 TI) x (64 TJ) output tile; each
//     wave owns (32 TI) x (32 TJ) outputs as TI x TJ int32 accumulators of
//     v_mfma_i32_32x32x32_i8.
//   * both operands are K-contiguous: each 128-wide K step copies the tile's
//     X and W rows (128 bytes each) from global memory straight into LDS
//     (global_load_lds_dwordx4) through a ring of S slots, S - 1 steps ahead.
//     LDS rows keep the XOR-swizzled chunk order of lds_copy.h.  The shipped
//     tiles: 64 x 64 (S = 2, 32 KiB) and 64 x 192 (S = 3, 96 KiB) for small
//     grids, 128 x 192 and 128 x 128 (S = 2, 80 and 64 KiB, two workgroups
//     per CU) for large ones.
//   * MFMA slice u (0..3) of a step, lane half h, covers k = 32 u + 16 h +
//     (0..15) for both operands (the MFMA sums over k, so any common
//     assignment is the same contraction): one conflict-free ds_read_b128 per
//     fragment, read while the previous slice's MFMAs run.
//   * the epilogue works on the accumulator registers: int32 -> fp32 (nearest
//     even) -> * x_scale -> * w_scale -> + bias -> bf16 (nearest even), with
//     the scales loaded before the main loop and adjacent columns paired into
//     dword stores; or the raw int32 for the accumulator-only entry point.
#include <hip/hip_runtime.h>

#include "lds_copy.h"
#include "q4k_device.h"
#include "q4k_launch.h"

namespace q4k {
namespace {

typedef int i4_t __attribute__((ext_vector_type(4)));
typedef int i16_t __attribute__((ext_vector_type(16)));

constexpr int kI8BK = 128;  // k per step = bytes per tile row and step

template <int TI, int TJ, int S>
struct W8Tile {
  static constexpr int BM = 64 * TI, BN = 64 * TJ;
  static constexpr int XBytes = BM * kI8BK, WBytes = BN * kI8BK;
  static constexpr int Slot = XBytes + WBytes;
  static constexpr int Lds = S * Slot;
  // 16-byte-per-lane copies per wave and step (one copy = 8 rows of 128 bytes)
  static constexpr int XC = BM / 32, WC = BN / 32, C = XC + WC;
  static_assert(S >= 2 && S <= 4, "ring of 2..4 slots");
  static_assert(Lds <= 160 * 1024, "LDS budget of one workgroup");
};

enum W8Out { kW8Acc = 0, kW8Bf16 = 1 };

// Wait until the copies of all but the last `pending` (0..2) issued steps
// have landed, then barrier.
template <int C>
__device__ __forceinline__ void wait_steps_barrier(int pending) {
  if (pending >= 2)
    wait_copies_barrier<2 * C>();
  else if (pending == 1)
    wait_copies_barrier<C>();
  else
    wait_copies_barrier<0>();
}

// The epilogue of one output: fp32 operations rounded one at a time.
// (The pragma keeps the compiler from contracting the last multiply and the
// add into one fma.)
__device__ __forceinline__ float w8_dequant(int acc, float xs, float ws, const float* bias,
                                            float b) {
#pragma clang fp contract(off)
  float a = static_cast<float>(acc) * xs;
  a = a * ws;
  if (bias) a = a + b;
  return a;
}

__device__ __forceinline__ uint32_t bf16_bits(float v) { return pack_bf16x2(v, v) & 0xFFFFu; }

// Exchange a dword with the neighbouring lane (lanes 2i and 2i+1 swap).
__device__ __forceinline__ uint32_t swap_lane_pairs(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1, 0xF, 0xF, true));  // quad_perm 1,0,3,2
}

// Workgroup = 4 waves as 2 x 2 over a (64 TI) x (64 TJ) output tile, each wave
// (32 TI) x (32 TJ) outputs as TI x TJ accumulators of v_mfma_i32_32x32x32_i8.
// K advances 128 per step; the tile's X and W rows of a step are copied
// straight into LDS slot s % S, S - 1 steps ahead, and a step's fragments are
// read slice by slice while the MFMAs of the previous slice run.
template <int TI, int TJ, int S, int OUT>
__global__ __launch_bounds__(256, 2) void k_w8a8_gemm(
    const int8_t* __restrict__ x, const int8_t* __restrict__ w, const float* __restrict__ xs,
    const float* __restrict__ ws, const float* __restrict__ bias, void* __restrict__ out, int m,
    int n, int k, int tiles_m, int tiles_n, int xcd_gm) {
  using T = W8Tile<TI, TJ, S>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[T::Lds];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int h = lane >> 5;
  const int c32 = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, xcd_gm, tm, tn);
  const int m0 = tm * T::BM, n0 = tn * T::BN;
  const int nst = k / kI8BK;
  // Output coordinates: accumulator r of a 32 x 32 tile holds row
  // 8 (r / 4) + 4 h + r % 4, column c32.
  const int row0 = m0 + 32 * TI * wm + 4 * h;
  const int col0 = n0 + 32 * TJ * wn + c32;

  // The epilogue's scales are loaded first (clamped indices, no branches):
  // their latency hides under the main loop.
  float xsr[TI][16], wsc[TJ], bv[TJ];
  if constexpr (OUT == kW8Bf16) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        xsr[i][r] = xs[min(row0 + 32 * i + 8 * (r >> 2) + (r & 3), m - 1)];
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      wsc[j] = ws[min(col0 + 32 * j, n - 1)];
      bv[j] = bias ? bias[min(col0 + 32 * j, n - 1)] : 0.0f;
    }
  }

  // Copy q of this wave fills tile rows 8 (wave C + q) .. +7: lane -> (row
  // lane / 8, LDS chunk lane % 8), which holds global chunk (lane % 8) ^ swz.
  // Rows past m or n re-read the last row (their results are not stored).
  const int8_t* xsrc[T::XC];
  const int8_t* wsrc[T::WC];
#pragma unroll
  for (int q = 0; q < T::XC; ++q) {
    const int row = 8 * (wave * T::XC + q) + (lane >> 3);
    xsrc[q] = x + static_cast<size_t>(min(m0 + row, m - 1)) * k + 16 * ((lane & 7) ^ swz(row));
  }
#pragma unroll
  for (int q = 0; q < T::WC; ++q) {
    const int row = 8 * (wave * T::WC + q) + (lane >> 3);
    wsrc[q] = w + static_cast<size_t>(min(n0 + row, n - 1)) * k + 16 * ((lane & 7) ^ swz(row));
  }
  const uint32_t lds0 = lds_address(smem);
  auto copy = [&](int s) {
    const uint32_t slot = lds0 + (s % S) * T::Slot;
    const size_t off = static_cast<size_t>(s) * kI8BK;
#pragma unroll
    for (int q = 0; q < T::XC; ++q)
      copy16_to_lds(xsrc[q] + off, __builtin_amdgcn_readfirstlane(slot + (wave * T::XC + q) * 1024));
#pragma unroll
    for (int q = 0; q < T::WC; ++q)
      copy16_to_lds(wsrc[q] + off, __builtin_amdgcn_readfirstlane(slot + T::XBytes +
                                                                  (wave * T::WC + q) * 1024));
  };

  // MFMA slice u (0..3) of a step, lane half h: k = 32 u + 16 h + (0..15) for
  // both operands, one ds_read_b128 per fragment.
  struct Frag {
    i4_t a[TI];
    i4_t b[TJ];
  };
  auto read = [&](int s, int u, Frag& F) {
    const uint8_t* base = smem + (s % S) * T::Slot;
    const int ch = 2 * u + h;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int r = 32 * TI * wm + 32 * i + c32;
      F.a[i] = *reinterpret_cast<const i4_t*>(base + r * kI8BK + ((ch ^ swz(r)) << 4));
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int r = 32 * TJ * wn + 32 * j + c32;
      F.b[j] = *reinterpret_cast<const i4_t*>(base + T::XBytes + r * kI8BK + ((ch ^ swz(r)) << 4));
    }
  };

  i16_t acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;
  auto mfmas = [&](const Frag& F) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(F.a[i], F.b[j], acc[i][j], 0, 0, 0);
  };

  // Prologue: copies of steps 0 .. S-2; step 0 lands.
  const int pre = min(nst, S - 1);
  for (int s = 0; s < pre; ++s) copy(s);
  wait_steps_barrier<T::C>(max(0, min(pre - 1, S - 2)));
  // Step s: refill slot (s - 1) % S, which every wave finished reading before
  // the last barrier, with step s + S - 1; the four slices of step s; then
  // step s + 1 lands (the copies issued after it may stay in flight) and the
  // barrier publishes it.
  for (int s = 0; s < nst; ++s) {
    if (s + S - 1 < nst) copy(s + S - 1);
    Frag F0, F1;
    read(s, 0, F0);
    read(s, 1, F1);
    mfmas(F0);
    read(s, 2, F0);
    mfmas(F1);
    read(s, 3, F1);
    mfmas(F0);
    mfmas(F1);
    wait_steps_barrier<T::C>(max(0, min(min(s + S - 1, nst - 1) - (s + 1), S - 2)));
  }

  if constexpr (OUT == kW8Bf16) {
    // Rows R and R + 1 of a column sit in one lane (elements r, r + 1); lanes
    // 2i and 2i + 1 hold adjacent columns.  Swapping one value between them
    // gives the even lane row R and the odd lane row R + 1, each as a pair of
    // adjacent bf16 stored as one dword (when n is even; otherwise one value
    // per store).
    uint16_t* const o16 = static_cast<uint16_t*>(out);
    const bool odd = (c32 & 1) != 0;
    const bool pairs = (n & 1) == 0;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int col = col0 + 32 * j;
#pragma unroll
      for (int i = 0; i < TI; ++i) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const int row = row0 + 32 * i + 8 * (r >> 2) + (r & 3);
          const uint32_t b0 = bf16_bits(w8_dequant(acc[i][j][r], xsr[i][r], wsc[j], bias, bv[j]));
          const uint32_t b1 =
              bf16_bits(w8_dequant(acc[i][j][r + 1], xsr[i][r + 1], wsc[j], bias, bv[j]));
          const uint32_t recv = swap_lane_pairs(odd ? b0 : b1);
          if (pairs) {
            const int rr = odd ? row + 1 : row;
            const uint32_t word = odd ? (recv | (b1 << 16)) : (b0 | (recv << 16));
            if (rr < m && col < n)
              *reinterpret_cast<uint32_t*>(o16 + static_cast<size_t>(rr) * n + (col & ~1)) = word;
          } else {
            if (row < m && col < n) o16[static_cast<size_t>(row) * n + col] = b0;
            if (row + 1 < m && col < n) o16[static_cast<size_t>(row + 1) * n + col] = b1;
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int col = col0 + 32 * j;
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = row0 + 32 * i + 8 * (r >> 2) + (r & 3);
          if (row < m && col < n) static_cast<int32_t*>(out)[static_cast<size_t>(row) * n + col] = acc[i][j][r];
        }
    }
  }
}

// Standalone epilogue: int32 [m, n] -> bf16 [m, n].  Thread -> VEC consecutive
// columns (VEC = 4 needs n % 4 == 0 and 16-byte aligned scales and bias);
// grid.y strides over the rows.
template <int VEC>
__global__ __launch_bounds__(256) void k_w8a8_epilogue(const int32_t* __restrict__ acc,
                                                       uint16_t* __restrict__ out,
                                                       const float* __restrict__ xs,
                                                       const float* __restrict__ ws,
                                                       const float* __restrict__ bias, int m,
                                                       int n) {
  const int col = (blockIdx.x * 256 + threadIdx.x) * VEC;
  if (col >= n) return;
  if constexpr (VEC == 4) {
    const float4 wv = *reinterpret_cast<const float4*>(ws + col);
    float4 bv = {0.0f, 0.0f, 0.0f, 0.0f};
    if (bias) bv = *reinterpret_cast<const float4*>(bias + col);
    for (int row = blockIdx.y; row < m; row += gridDim.y) {
      const size_t o = static_cast<size_t>(row) * n + col;
      const float xsr = xs[row];
      const int4 a = *reinterpret_cast<const int4*>(acc + o);
      const float y0 = w8_dequant(a.x, xsr, wv.x, bias, bv.x);
      const float y1 = w8_dequant(a.y, xsr, wv.y, bias, bv.y);
      const float y2 = w8_dequant(a.z, xsr, wv.z, bias, bv.z);
      const float y3 = w8_dequant(a.w, xsr, wv.w, bias, bv.w);
      *reinterpret_cast<uint2*>(out + o) = uint2{pack_bf16x2(y0, y1), pack_bf16x2(y2, y3)};
    }
  } else {
    const float wv = ws[col];
    const float bv = bias ? bias[col] : 0.0f;
    for (int row = blockIdx.y; row < m; row += gridDim.y) {
      const size_t o = static_cast<size_t>(row) * n + col;
      out[o] = bf16_bits(w8_dequant(acc[o], xs[row], wv, bias, bv));
    }
  }
}

// Row quantizer: one wave per row of bf16 [rows, k] (k % 8 == 0): amax over
// the row (wave max), scale = amax / 127, codes = clamp(rint(v / scale)).
// Lane l handles the 8-element groups l, l + 64, ...  With G > 0 (k <= 512 G)
// a lane loads all its groups at once and keeps them in registers for the
// second pass; with G = 0 it walks the row twice (the second pass from cache),
// for any k.
__device__ __forceinline__ void bf16_pair(uint32_t v, float& lo, float& hi) {
  lo = __builtin_bit_cast(float, v << 16);
  hi = __builtin_bit_cast(float, v & 0xFFFF0000u);
}

__device__ __forceinline__ float group_amax(uint4 v, float amax) {
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float lo, hi;
    bf16_pair(u[e], lo, hi);
    amax = fmaxf(amax, fmaxf(fabsf(lo), fabsf(hi)));
  }
  return amax;
}

// Codes of one 8-element group: rint(v / s) clamped to +-127 (0 when s = 0).
__device__ __forceinline__ uint2 group_codes(uint4 v, float s) {
  const uint32_t u[4] = {v.x, v.y, v.z, v.w};
  uint32_t packed[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float f[2];
    bf16_pair(u[e], f[0], f[1]);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      int c = 0;
      if (s != 0.0f) {
        const float r = fminf(fmaxf(__builtin_rintf(__fdiv_rn(f[p], s)), -127.0f), 127.0f);
        c = static_cast<int>(r);
      }
      packed[e >> 1] |= (static_cast<uint32_t>(c) & 0xFFu) << (8 * (2 * (e & 1) + p));
    }
  }
  return uint2{packed[0], packed[1]};
}

template <int G>
__global__ __launch_bounds__(256) void k_w8a8_quantize_rows(const uint16_t* __restrict__ x,
                                                            int8_t* __restrict__ q,
                                                            float* __restrict__ scale, int rows,
                                                            int k) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // uniform per wave; no barrier below
  const uint16_t* xr = x + static_cast<size_t>(row) * k;
  int8_t* qr = q + static_cast<size_t>(row) * k;
  const int groups = k >> 3;
  float amax = 0.0f;
  uint4 v[G > 0 ? G : 1];
  if constexpr (G > 0) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int g = lane + 64 * i;
      v[i] = g < groups ? *reinterpret_cast<const uint4*>(xr + 8 * g) : uint4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < G; ++i) amax = group_amax(v[i], amax);
  } else {
    for (int g = lane; g < groups; g += 64)
      amax = group_amax(*reinterpret_cast<const uint4*>(xr + 8 * g), amax);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 64));
  const float s = __fdiv_rn(amax, 127.0f);
  if (lane == 0) scale[row] = s;
  if constexpr (G > 0) {
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const int g = lane + 64 * i;
      if (g < groups) *reinterpret_cast<uint2*>(qr + 8 * g) = group_codes(v[i], s);
    }
  } else {
    for (int g = lane; g < groups; g += 64)
      *reinterpret_cast<uint2*>(qr + 8 * g) = group_codes(*reinterpret_cast<const uint4*>(xr + 8 * g), s);
  }
}

template <int TI, int TJ, int S, int OUT>
hipError_t launch_tiles(const int8_t* x, const int8_t* w, const float* xs, const float* ws,
                        const float* bias, void* out, int m, int n, int k, hipStream_t stream) {
  using T = W8Tile<TI, TJ, S>;
  const int tiles_m = (m + T::BM - 1) / T::BM, tiles_n = (n + T::BN - 1) / T::BN;
  const int gm = xcd_blocking(tiles_m, tiles_n, static_cast<long>(T::XBytes),
                              static_cast<long>(T::WBytes));
  hipLaunchKernelGGL((k_w8a8_gemm<TI, TJ, S, OUT>), dim3(tiles_m * tiles_n), dim3(256), 0, stream,
                     x, w, xs, ws, bias, out, m, n, k, tiles_m, tiles_n, gm);
  return hipGetLastError();
}

}  // namespace

namespace {

// Tile shape per grid.  The loop is bound by the L2 read requests a CU can
// keep in flight (about 70 128-byte lines; counters: the TCP waits on L2 data
// half its cycles while the MFMA pipe is 30% busy), so the wider the tile,
// the fewer requests per MAC.  N-wide 192 tiles are used where they pad N no
// more than 128-wide ones do.  3072 x 3072 weights, warm timings:
//   * grids up to 256 tiles of 128 x 128 (M = 512 / 1024): 64 x 192 tiles
//     with a three-slot ring (96 KiB, one workgroup per CU) where they still
//     give every CU one (M = 1024: 23.5 us against 25.9 for 64 x 64 and 27
//     for 64 x 128), else 64 x 64 (two slots, several per CU);
//   * larger grids: 128 x 192 with two slots (80 KiB, two workgroups per CU;
//     M = 8192: 99 us against 111 for 128 x 128, which remains for other N).
//     Tiles that leave one workgroup per CU lose even with fewer requests
//     (256 x 192: 110 us; 256 x 128 three slots: 122; 128 x 128 three or four
//     slots: 134), as do 64-byte K steps, which halve the request size.
template <int OUT>
hipError_t launch_w8a8(const int8_t* x, const int8_t* w, const float* xs, const float* ws,
                       const float* bias, void* out, int64_t m, int64_t n, int64_t k,
                       hipStream_t stream) {
  const int mi = static_cast<int>(m), ni = static_cast<int>(n), ki = static_cast<int>(k);
  const int64_t tiles128 = ((m + 127) / 128) * ((n + 127) / 128);
  const bool n192 = (n + 191) / 192 * 192 <= (n + 127) / 128 * 128;
  if (tiles128 <= 256) {
    if (n192 && ((m + 63) / 64) * ((n + 191) / 192) >= 256)
      return launch_tiles<1, 3, 3, OUT>(x, w, xs, ws, bias, out, mi, ni, ki, stream);
    return launch_tiles<1, 1, 2, OUT>(x, w, xs, ws, bias, out, mi, ni, ki, stream);
  }
  if (n192) return launch_tiles<2, 3, 2, OUT>(x, w, xs, ws, bias, out, mi, ni, ki, stream);
  return launch_tiles<2, 2, 2, OUT>(x, w, xs, ws, bias, out, mi, ni, ki, stream);
}

}  // namespace

hipError_t launch_w8a8_linear(const int8_t* x, const float* x_scale, const int8_t* w,
                              const float* w_scale, const float* bias, uint16_t* out, int64_t m,
                              int64_t n, int64_t k, hipStream_t stream) {
  return launch_w8a8<kW8Bf16>(x, w, x_scale, w_scale, bias, out, m, n, k, stream);
}

hipError_t launch_w8a8_linear_acc(const int8_t* x, const int8_t* w, int32_t* acc, int64_t m,
                                  int64_t n, int64_t k, hipStream_t stream) {
  return launch_w8a8<kW8Acc>(x, w, nullptr, nullptr, nullptr, acc, m, n, k, stream);
}

hipError_t launch_w8a8_epilogue(const int32_t* acc, uint16_t* out, const float* x_scale,
                                const float* w_scale, const float* bias, int64_t m, int64_t n,
                                hipStream_t stream) {
  const int mi = static_cast<int>(m), ni = static_cast<int>(n);
  const bool vec = ni % 4 == 0 && (reinterpret_cast<uintptr_t>(w_scale) & 15u) == 0 &&
                   (bias == nullptr || (reinterpret_cast<uintptr_t>(bias) & 15u) == 0);
  const int per = vec ? 4 : 1;
  const int cols = (ni + per - 1) / per;
  const dim3 grid(static_cast<unsigned>((cols + 255) / 256), static_cast<unsigned>(min(mi, 4096)));
  if (vec)
    hipLaunchKernelGGL((k_w8a8_epilogue<4>), grid, dim3(256), 0, stream, acc, out, x_scale,
                       w_scale, bias, mi, ni);
  else
    hipLaunchKernelGGL((k_w8a8_epilogue<1>), grid, dim3(256), 0, stream, acc, out, x_scale,
                       w_scale, bias, mi, ni);
  return hipGetLastError();
}

hipError_t launch_w8a8_quantize_rows(const uint16_t* x, int8_t* q, float* scale, int64_t rows,
                                     int64_t k, hipStream_t stream) {
  const int r = static_cast<int>(rows), ki = static_cast<int>(k);
  const dim3 grid((r + 3) / 4);
  if (ki <= 64 * 8 * 8)
    hipLaunchKernelGGL((k_w8a8_quantize_rows<8>), grid, dim3(256), 0, stream, x, q, scale, r, ki);
  else if (ki <= 64 * 8 * 16)
    hipLaunchKernelGGL((k_w8a8_quantize_rows<16>), grid, dim3(256), 0, stream, x, q, scale, r, ki);
  else
    hipLaunchKernelGGL((k_w8a8_quantize_rows<0>), grid, dim3(256), 0, stream, x, q, scale, r, ki);
  return hipGetLastError();
}

}  // namespace q4k
