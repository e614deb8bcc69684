// k_planes.hip -- the k-quants that keep their high bits in a separate plane,
// Q6_K and Q3_K: decode GEMV and the dequant export.
//
// Formats (the daScript PR page "CPU kernel parity: decode and tile kernels
// at llama.cpp speed ..." names "k6" and "k3": their high bits live in planes
// beside the low bits and one scale per 16-weight sub-block is flushed into
// the accumulator; the layouts are the GGUF reading, the pages print none).
// Weight i = 128h + 32j + l (h = 0..1, j = 0..3, l = 0..31), sub-block i / 16:
//   Q6_K, 210 bytes: ql[128] at 0, qh[64] at 128, signed 8-bit scales sc[16]
//     at 192, fp16 d at 208.  q = low (j < 2) or high (j >= 2) nibble of
//     ql[64h + 32(j mod 2) + l] + 16 * (bits 2j, 2j+1 of qh[32h + l]);
//     w = d * sc[i/16] * (q - 32).
//   Q3_K, 110 bytes: hmask[32] at 0, qs[64] at 32, 12 bytes of packed 6-bit
//     scales at 96, fp16 d at 108.  q = bits 2j, 2j+1 of qs[32h + l]
//     + 4 * (bit 4h + j of hmask[l]); sub-block t's scale u_t has the low
//     (t < 8) or high (t >= 8) nibble of byte t mod 8 and bits 2(t/4),
//     2(t/4)+1 of byte 8 + t mod 4 on top; w = d * (u_t - 32) * (q - 4).
//
// Design for gfx950:
//   * A unit is (block, h, c): the 32 weights 128h + 32j + 8c + e (j = 0..3,
//     e = 0..7), whose 8 bytes of each low-bit and high-bit field start at a
//     multiple of 8 inside the block.  Four quants of one j come out of a
//     pair of dwords with masks, shifts and an OR, in the bytes' order; the
//     unit's four sub-block scales are decoded to d * sc (exact in fp32).
//   * Both block sizes are 2 (mod 4), so a block starts 0 or 2 bytes past a
//     dword boundary (the matrix itself is 16-byte aligned).  Every field read
//     sits at a multiple of 4 inside the block: it is read as the aligned
//     dwords below it (one more when the block is 2 bytes off) and
//     v_alignbyte shifts the bytes into place.  No read leaves the block; d
//     is one 16-bit load.
//   * The scale multiplies sums of 8 weights: per unit and j the GEMV forms
//     dot = sum q x and s8 = sum x in fp32 and adds (d sc) (dot - OFF s8)
//     (OFF = 32 or 4), so the quant offset costs one FMA per 8 weights.
//   * GEMV: 8 waves per workgroup, 2 rows per wave (16 rows per workgroup;
//     measured against 4x4, 8x4, 16x1, 4x2 and 8x1, it was 8-14% faster than
//     4x4 on 4096- and 14336-row matrices).  Per 4096-wide chunk of x a lane
//     owns units lane and lane + 64; it issues the chunk's weight loads first,
//     then x is staged once per workgroup in LDS and each lane copies its
//     units' x values and 8-sums into registers, reused for both rows.
//     Batches run in passes of up to 4 x rows: each unit's quants are widened
//     once per pass and serve every x row.
//   * Dequant export: one thread per unit, fp32 = (d sc) * (q - OFF) (the
//     exact weight rounded once) or its bf16 (nearest even).
#include <hip/hip_runtime.h>

#include "q4k_device.h"
#include "q4k_launch.h"

namespace q4k {
namespace {

constexpr int kPlaneChunk = 4096;  // x elements staged per pass (16 KiB)
constexpr int kPlaneUnitsPerLane = kPlaneChunk / 32 / 64;

// Up to four dwords read from the dword boundary at or below p (p = the
// field's address, s = p mod 4 in {0, 2}); the last one only when s = 2.
template <int N>
__device__ __forceinline__ void load_field(const uint8_t* p, uint32_t s, uint32_t (&f)[N + 1]) {
  const uint32_t* a = reinterpret_cast<const uint32_t*>(p - s);
#pragma unroll
  for (int i = 0; i < N; ++i) f[i] = a[i];
  f[N] = 0u;
  if (s) f[N] = a[N];
}

// v_alignbyte_b32(hi, lo, n) = the 64-bit {hi, lo} shifted right by n bytes.
template <int N>
__device__ __forceinline__ void align_field(const uint32_t (&f)[N + 1], uint32_t s,
                                            uint32_t (&v)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = __builtin_amdgcn_alignbyte(f[i + 1], f[i], s);
}

// The decoded unit: quants q[j][e / 4] (four values per dword, weight e in
// byte e % 4, offset by OFF) and the four scales d * sc.
struct PlaneUnit {
  uint32_t q[4][2];
  float dsc[4];
};

template <int FMT>
struct Planes;

template <>
struct Planes<6> {
  static constexpr int Bytes = 210;
  static constexpr float Off = 32.0f;
  struct Raw {
    uint32_t lo[3], hi[3], qh[3], sc[3];
    uint32_t d, s;
  };
  static __device__ __forceinline__ Raw load(const uint8_t* blk, int h, int c) {
    Raw r;
    r.s = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(blk) & 3u);
    load_field<2>(blk + 64 * h + 8 * c, r.s, r.lo);
    load_field<2>(blk + 64 * h + 32 + 8 * c, r.s, r.hi);
    load_field<2>(blk + 128 + 32 * h + 8 * c, r.s, r.qh);
    load_field<2>(blk + 192 + 8 * h, r.s, r.sc);
    r.d = *reinterpret_cast<const uint16_t*>(blk + 208);
    return r;
  }
  static __device__ __forceinline__ PlaneUnit decode(const Raw& r, int h, int c) {
    uint32_t L[2], H[2], Q[2], S[2];
    align_field<2>(r.lo, r.s, L);
    align_field<2>(r.hi, r.s, H);
    align_field<2>(r.qh, r.s, Q);
    align_field<2>(r.sc, r.s, S);
    PlaneUnit u;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      u.q[0][e] = (L[e] & 0x0F0F0F0Fu) | ((Q[e] << 4) & 0x30303030u);
      u.q[1][e] = (H[e] & 0x0F0F0F0Fu) | ((Q[e] << 2) & 0x30303030u);
      u.q[2][e] = ((L[e] >> 4) & 0x0F0F0F0Fu) | (Q[e] & 0x30303030u);
      u.q[3][e] = ((H[e] >> 4) & 0x0F0F0F0Fu) | ((Q[e] >> 2) & 0x30303030u);
    }
    const float d = half_bits_to_float(r.d);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = 2 * j + (c >> 1);  // scale byte of the half: sub-block 8h + 2j + c/2
      const uint32_t word = b < 4 ? S[0] : S[1];
      u.dsc[j] = d * static_cast<float>(static_cast<int8_t>((word >> (8 * (b & 3))) & 0xFFu));
    }
    (void)h;
    return u;
  }
};

template <>
struct Planes<3> {
  static constexpr int Bytes = 110;
  static constexpr float Off = 4.0f;
  struct Raw {
    uint32_t hm[3], qs[3], sc[4];
    uint32_t d, s;
  };
  static __device__ __forceinline__ Raw load(const uint8_t* blk, int h, int c) {
    Raw r;
    r.s = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(blk) & 3u);
    load_field<2>(blk + 8 * c, r.s, r.hm);
    load_field<2>(blk + 32 + 32 * h + 8 * c, r.s, r.qs);
    load_field<3>(blk + 96, r.s, r.sc);
    r.d = *reinterpret_cast<const uint16_t*>(blk + 108);
    return r;
  }
  static __device__ __forceinline__ PlaneUnit decode(const Raw& r, int h, int c) {
    uint32_t Hm[2], Qs[2], S[3];
    align_field<2>(r.hm, r.s, Hm);
    align_field<2>(r.qs, r.s, Qs);
    align_field<3>(r.sc, r.s, S);
    PlaneUnit u;
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        u.q[j][e] = ((Qs[e] >> (2 * j)) & 0x03030303u) |
                    (((Hm[e] >> (4 * h + j)) & 0x01010101u) << 2);
    const float d = half_bits_to_float(r.d);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // sub-block t = 8h + 2j + c/2: low nibble (h = 0) or high nibble (h = 1)
      // of scale byte b = 2j + c/2; top bits 2(t/4), 2(t/4)+1 of byte 8 + b % 4
      const int b = 2 * j + (c >> 1);
      const uint32_t low4 = ((b < 4 ? S[0] : S[1]) >> (8 * (b & 3) + 4 * h)) & 15u;
      const uint32_t top2 = (S[2] >> (8 * (b & 3) + 2 * (2 * h + (j >> 1)))) & 3u;
      u.dsc[j] = d * static_cast<float>(static_cast<int>(low4 | (top2 << 4)) - 32);
    }
    return u;
  }
};

// WAVES waves per workgroup, RPW rows per wave, up to MT rows of x per pass
// (mrows of them used): each unit's quants are decoded and widened once and
// serve every x row.
template <int FMT, int WAVES, int RPW, int MT>
__global__ __launch_bounds__(64 * WAVES) void k_gemv_planes(const uint8_t* __restrict__ w,
                                                            const float* __restrict__ x,
                                                            float* __restrict__ y, int n, int k,
                                                            int mrows) {
  using P = Planes<FMT>;
  __shared__ __attribute__((aligned(16))) float xs[MT][kPlaneChunk];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row0 = (blockIdx.x * WAVES + wave) * RPW;
  const size_t row_bytes = static_cast<size_t>(k >> 8) * P::Bytes;
  const uint8_t* rows[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
    rows[r] = w + static_cast<size_t>(min(row0 + r, n - 1)) * row_bytes;
  float acc[MT][RPW];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int r = 0; r < RPW; ++r) acc[i][r] = 0.0f;

  for (int c0 = 0; c0 < k; c0 += kPlaneChunk) {
    const int kc = min(kPlaneChunk, k - c0);  // a multiple of 256
    const int units = kc >> 5;                // 8 per block
    // Units past a short chunk's end re-read its last unit (not accumulated).
    typename P::Raw raw[kPlaneUnitsPerLane][RPW];
#pragma unroll
    for (int t = 0; t < kPlaneUnitsPerLane; ++t) {
      const int u = min(lane + 64 * t, units - 1);
      const int bg = (c0 >> 8) + (u >> 3);
#pragma unroll
      for (int r = 0; r < RPW; ++r)
        raw[t][r] = P::load(rows[r] + static_cast<size_t>(bg) * P::Bytes, (u >> 2) & 1, u & 3);
    }
    __syncthreads();  // the previous chunk's reads of xs are done
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      if (i >= mrows) break;
      for (int e = 4 * static_cast<int>(threadIdx.x); e < kc; e += 4 * 64 * WAVES)
        *reinterpret_cast<float4*>(&xs[i][e]) =
            *reinterpret_cast<const float4*>(x + static_cast<size_t>(i) * k + c0 + e);
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < kPlaneUnitsPerLane; ++t) {
      const int u = lane + 64 * t;
      if (u >= units) continue;
      const int bl = u >> 3, h = (u >> 2) & 1, c = u & 3;
      PlaneUnit wu[RPW];
#pragma unroll
      for (int r = 0; r < RPW; ++r) wu[r] = P::decode(raw[t][r], h, c);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float qf[RPW][8];
#pragma unroll
        for (int r = 0; r < RPW; ++r)
#pragma unroll
          for (int e = 0; e < 8; ++e) qf[r][e] = ubyte_f32(wu[r].q[j][e >> 2], e & 3);
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          if (i >= mrows) break;
          const float* p = &xs[i][256 * bl + 128 * h + 32 * j + 8 * c];
          const float4 a = *reinterpret_cast<const float4*>(p);
          const float4 b = *reinterpret_cast<const float4*>(p + 4);
          const float xv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
          const float s8 = ((a.x + a.y) + (a.z + a.w)) + ((b.x + b.y) + (b.z + b.w));
#pragma unroll
          for (int r = 0; r < RPW; ++r) {
            float dot = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) dot = fmaf(qf[r][e], xv[e], dot);
            acc[i][r] = fmaf(wu[r].dsc[j], fmaf(-P::Off, s8, dot), acc[i][r]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const float v = wave_sum(acc[i][r]);
      if (lane == 0 && i < mrows && row0 + r < n) y[static_cast<size_t>(i) * n + row0 + r] = v;
    }
}

// One thread per unit of the matrix (8 per block, blocks in row-major order).
template <int FMT, bool BF16>
__global__ __launch_bounds__(256) void k_dequant_planes(const uint8_t* __restrict__ w,
                                                        void* __restrict__ out, int64_t units) {
  using P = Planes<FMT>;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= units) return;
  const int64_t g = t >> 3;  // global block index = row * (k / 256) + b
  const int h = static_cast<int>((t >> 2) & 1), c = static_cast<int>(t & 3);
  const PlaneUnit u = P::decode(P::load(w + g * P::Bytes, h, c), h, c);
  // block g covers output elements 256 g .. 256 g + 255 of the row-major [n, k]
  const int64_t base = 256 * g + 128 * h + 8 * c;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = u.dsc[j] * (ubyte_f32(u.q[j][e >> 2], e & 3) - P::Off);
    if constexpr (BF16) {
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + base + 32 * j) =
          uint4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                pack_bf16x2(v[6], v[7])};
    } else {
      float* o = static_cast<float*>(out) + base + 32 * j;
      *reinterpret_cast<float4*>(o) = float4{v[0], v[1], v[2], v[3]};
      *reinterpret_cast<float4*>(o + 4) = float4{v[4], v[5], v[6], v[7]};
    }
  }
}

// Batches run in passes of up to 4 x rows (W is streamed once per pass).
template <int FMT, int WAVES = 8, int RPW = 2>
hipError_t launch_gemv_planes(const uint8_t* w, const float* x, float* y, int64_t m, int64_t n,
                              int64_t k, hipStream_t stream) {
  const int ni = static_cast<int>(n), ki = static_cast<int>(k);
  const int rows_per_wg = WAVES * RPW;
  const dim3 grid(static_cast<unsigned>((ni + rows_per_wg - 1) / rows_per_wg));
  for (int64_t i0 = 0; i0 < m; i0 += 4) {
    const int mm = static_cast<int>(m - i0 < 4 ? m - i0 : 4);
    const float* xs = x + i0 * k;
    float* ys = y + i0 * n;
    if (mm == 1)
      hipLaunchKernelGGL((k_gemv_planes<FMT, WAVES, RPW, 1>), grid, dim3(64 * WAVES), 0, stream,
                         w, xs, ys, ni, ki, mm);
    else if (mm == 2)
      hipLaunchKernelGGL((k_gemv_planes<FMT, WAVES, RPW, 2>), grid, dim3(64 * WAVES), 0, stream,
                         w, xs, ys, ni, ki, mm);
    else
      hipLaunchKernelGGL((k_gemv_planes<FMT, WAVES, RPW, 4>), grid, dim3(64 * WAVES), 0, stream,
                         w, xs, ys, ni, ki, mm);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int FMT, bool BF16>
hipError_t launch_dequant_planes(const uint8_t* w, void* out, int64_t n, int64_t k,
                                 hipStream_t stream) {
  const int64_t units = n * (k / 256) * 8;
  hipLaunchKernelGGL((k_dequant_planes<FMT, BF16>),
                     dim3(static_cast<unsigned>((units + 255) / 256)), dim3(256), 0, stream, w,
                     out, units);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_q6k_gemv(const uint8_t* w, const float* x, float* y, int64_t m, int64_t n,
                           int64_t k, hipStream_t stream) {
  return launch_gemv_planes<6>(w, x, y, m, n, k, stream);
}
hipError_t launch_q6k_dequant_f32(const uint8_t* w, float* out, int64_t n, int64_t k,
                                  hipStream_t stream) {
  return launch_dequant_planes<6, false>(w, out, n, k, stream);
}
hipError_t launch_q6k_dequant_bf16(const uint8_t* w, uint16_t* out, int64_t n, int64_t k,
                                   hipStream_t stream) {
  return launch_dequant_planes<6, true>(w, out, n, k, stream);
}

hipError_t launch_q3k_gemv(const uint8_t* w, const float* x, float* y, int64_t m, int64_t n,
                           int64_t k, hipStream_t stream) {
  return launch_gemv_planes<3>(w, x, y, m, n, k, stream);
}
hipError_t launch_q3k_dequant_f32(const uint8_t* w, float* out, int64_t n, int64_t k,
                                  hipStream_t stream) {
  return launch_dequant_planes<3, false>(w, out, n, k, stream);
}
hipError_t launch_q3k_dequant_bf16(const uint8_t* w, uint16_t* out, int64_t n, int64_t k,
                                   hipStream_t stream) {
  return launch_dequant_planes<3, true>(w, out, n, k, stream);
}

}  // namespace q4k
