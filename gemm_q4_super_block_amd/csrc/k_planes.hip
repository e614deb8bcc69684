// k_planes.hip -- the k-quants that keep their high bits in a separate plane,
// Q6_K and Q3_K: decode GEMV, prefill GEMM and the dequant export.
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
//     v_alignbyte shifts the bytes into place.  A read starts at most 2 bytes
//     before its field (the previous block's tail: a block 2 bytes off is
//     never the matrix's first) and ends at most 2 bytes past it, inside the
//     block; d is one 16-bit load.
//   * The scale multiplies sums of 8 weights: per unit and j the GEMV forms
//     dot = sum (q - OFF) x in fp32 and adds (d sc) dot (OFF = 32 or 4).  q -
//     OFF is an exact small integer, so a zero weight adds exactly zero; the
//     offset is not applied to a separate sum of x, whose rounding would not
//     cancel against that of sum q x when the weights do.
//   * (q - OFF) is widened by one sign-extending byte convert: the quant
//     field with its top bit flipped is its two's-complement value, and
//     shifted to the top of its byte it reads as (q - OFF) * SCALE (SCALE =
//     4 for the 6-bit, 32 for the 3-bit fields), with SCALE taken off d sc.
//     Scaling by a power of two commutes with every rounding, so the sums
//     and the dequant export are what they would be unscaled.  Against an
//     unsigned convert and a subtraction per weight this is ~20% fewer VALU
//     instructions, and the batch-1 GEMVs are bound by them (4096 x 4096:
//     Q6_K 6.3-6.4 us against 8.0, Q3_K 6.2 against 7.4, with the shape
//     below).
//   * GEMV at batch 1: one row per wave, 4 waves per workgroup; x staged by
//     direct global -> LDS copies issued before the weight copies.  Passes of
//     2 to 4 x rows: 8 waves, 2 rows per wave, x staged by loads.  Per
//     4096-wide chunk of x a lane owns units lane and lane + 64; it issues
//     the chunk's weight loads first.  Each unit's quants are widened once
//     per pass and serve every x row (and both rows' dots).
//   * Dequant export: one thread per unit, fp32 = (d sc) * (q - OFF) (the
//     exact weight rounded once) or its bf16 (nearest even).
#include <hip/hip_runtime.h>

#include "lds_copy.h"
#include "q4k_device.h"
#include "q4k_launch.h"

namespace q4k {
namespace {

constexpr int kPlaneChunk = 4096;  // x elements staged per pass (16 KiB)
constexpr int kPlaneUnitsPerLane = kPlaneChunk / 32 / 64;
constexpr int kPlaneDecodeWaves = 4;  // waves (rows) per workgroup of the batch-1 GEMV

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

// The decoded unit: quants q[j][e / 4] (four per dword, weight e in byte
// e % 4) as the signed bytes (q - OFF) * SCALE, and the four scales
// d * sc / SCALE.  (q - OFF) is the quant field read as a two's-complement
// number after flipping its top bit; shifted to the top of its byte, one
// sign-extending byte convert per weight widens it, and SCALE (a power of
// two) comes off the scale exactly, so d sc (q - OFF) and every sum of its
// products are what they would be unscaled.
struct PlaneUnit {
  uint32_t q[4][2];
  float dsc[4];
};

// Byte i of v as a signed integer, exactly as a float.
__device__ __forceinline__ float sbyte_f32(uint32_t v, int i) {
  return static_cast<float>(static_cast<int8_t>((v >> (8 * i)) & 0xFFu));
}

template <int FMT>
struct Planes;

template <>
struct Planes<6> {
  static constexpr int Bytes = 210;
  static constexpr float Off = 32.0f;
  static constexpr float Scale = 4.0f;  // 6-bit fields: (q ^ 32) << 2
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
      u.q[0][e] = (((L[e] & 0x0F0F0F0Fu) | ((Q[e] << 4) & 0x30303030u)) ^ 0x20202020u) << 2;
      u.q[1][e] = (((H[e] & 0x0F0F0F0Fu) | ((Q[e] << 2) & 0x30303030u)) ^ 0x20202020u) << 2;
      u.q[2][e] = ((((L[e] >> 4) & 0x0F0F0F0Fu) | (Q[e] & 0x30303030u)) ^ 0x20202020u) << 2;
      u.q[3][e] = ((((H[e] >> 4) & 0x0F0F0F0Fu) | ((Q[e] >> 2) & 0x30303030u)) ^ 0x20202020u) << 2;
    }
    const float d = half_bits_to_float(r.d);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = 2 * j + (c >> 1);  // scale byte of the half: sub-block 8h + 2j + c/2
      const uint32_t word = b < 4 ? S[0] : S[1];
      u.dsc[j] = d * static_cast<float>(static_cast<int8_t>((word >> (8 * (b & 3))) & 0xFFu)) *
                 (1.0f / Scale);
    }
    (void)h;
    return u;
  }
};

template <>
struct Planes<3> {
  static constexpr int Bytes = 110;
  static constexpr float Off = 4.0f;
  static constexpr float Scale = 32.0f;  // 3-bit fields: (q ^ 4) << 5
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
        u.q[j][e] = ((((Qs[e] >> (2 * j)) & 0x03030303u) |
                     (((Hm[e] >> (4 * h + j)) & 0x01010101u) << 2)) ^ 0x04040404u) << 5;
    const float d = half_bits_to_float(r.d);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // sub-block t = 8h + 2j + c/2: low nibble (h = 0) or high nibble (h = 1)
      // of scale byte b = 2j + c/2; top bits 2(t/4), 2(t/4)+1 of byte 8 + b % 4
      const int b = 2 * j + (c >> 1);
      const uint32_t low4 = ((b < 4 ? S[0] : S[1]) >> (8 * (b & 3) + 4 * h)) & 15u;
      const uint32_t top2 = (S[2] >> (8 * (b & 3) + 2 * (2 * h + (j >> 1)))) & 3u;
      u.dsc[j] = d * static_cast<float>(static_cast<int>(low4 | (top2 << 4)) - 32) * (1.0f / Scale);
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
          for (int e = 0; e < 8; ++e) qf[r][e] = sbyte_f32(wu[r].q[j][e >> 2], e & 3);
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          if (i >= mrows) break;
          const float* p = &xs[i][256 * bl + 128 * h + 32 * j + 8 * c];
          const float4 a = *reinterpret_cast<const float4*>(p);
          const float4 b = *reinterpret_cast<const float4*>(p + 4);
          const float xv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
          for (int r = 0; r < RPW; ++r) {
            float dot = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) dot = fmaf(qf[r][e], xv[e], dot);
            acc[i][r] = fmaf(wu[r].dsc[j], dot, acc[i][r]);
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
// The same GEMV with each wave's weight rows staged through LDS: per K chunk
// a wave copies the chunk's bytes of its RPW rows (one contiguous range per
// row, from the 16-byte boundary at or below its start) straight into its own
// part of LDS with 16-byte-per-lane copies, and the units are then read from
// LDS exactly as the kernel above reads them from memory (the LDS copy keeps
// each byte's address mod 16).  A row's records are fetched by a few wide,
// contiguous loads instead of four to five small loads per unit.  The copied
// range ends at most 15 bytes past the chunk, so the host takes this kernel
// only when the matrix ends on a 16-byte boundary (n * k / 256 a multiple
// of 8).
template <int FMT>
struct PlaneRows {
  static constexpr int Units = (kPlaneChunk / 256 * Planes<FMT>::Bytes + 14 + 15) / 16;
  static constexpr int Copies = (Units + 63) / 64;  // 16-byte-per-lane copies per row
  static constexpr int Lds = Copies * 1024;          // LDS bytes per row
};

template <int FMT, int WAVES, int RPW, int MT>
__global__ __launch_bounds__(64 * WAVES) void k_gemv_planes_lds(const uint8_t* __restrict__ w,
                                                                const float* __restrict__ x,
                                                                float* __restrict__ y, int n,
                                                                int k, int mrows) {
  using P = Planes<FMT>;
  using RL = PlaneRows<FMT>;
  __shared__ __attribute__((aligned(16))) float xs[MT][kPlaneChunk];
  __shared__ __attribute__((aligned(16))) uint8_t wl[WAVES][RPW][RL::Lds];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
    const int cbytes = (kc >> 8) * P::Bytes;
    if (c0 > 0) __syncthreads();  // the previous chunk's reads of xs are done
    if constexpr (MT == 1) {
      // x by direct copies, issued first: 16-byte unit p of the chunk to LDS
      // unit p (units past the chunk repeat its last; never read).
#pragma unroll
      for (int q = 0; q < kPlaneChunk / 4 / (64 * WAVES); ++q) {
        const int p = 64 * (wave + WAVES * q) + lane;
        copy16_to_lds(x + c0 + 4 * min(p, (kc >> 2) - 1),
                      __builtin_amdgcn_readfirstlane(lds_address(&xs[0][0]) +
                                                     1024u * static_cast<uint32_t>(wave + WAVES * q)));
      }
    }
    // Row r's chunk: bytes [g0, g0 + cbytes) copied from a = g0 rounded down
    // to 16; unit u of the copy lands at LDS offset 16 u (units past the
    // range repeat its last unit).
    int off[RPW];
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const uint8_t* g0 = rows[r] + static_cast<size_t>(c0 >> 8) * P::Bytes;
      const uint8_t* a = reinterpret_cast<const uint8_t*>(reinterpret_cast<uintptr_t>(g0) & ~uintptr_t(15));
      off[r] = static_cast<int>(g0 - a);
      const int nu = (off[r] + cbytes + 15) >> 4;
      const uint32_t dst = lds_address(&wl[wave][r][0]);
#pragma unroll
      for (int q = 0; q < RL::Copies; ++q)
        copy16_to_lds(a + 16 * min(64 * q + lane, nu - 1),
                      __builtin_amdgcn_readfirstlane(dst + 1024 * q));
    }
    if constexpr (MT > 1) {
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        if (i >= mrows) break;
        for (int e = 4 * static_cast<int>(threadIdx.x); e < kc; e += 4 * 64 * WAVES)
          *reinterpret_cast<float4*>(&xs[i][e]) =
              *reinterpret_cast<const float4*>(x + static_cast<size_t>(i) * k + c0 + e);
      }
    }
    wait_copies_barrier<0>();
#pragma unroll
    for (int t = 0; t < kPlaneUnitsPerLane; ++t) {
      const int u = lane + 64 * t;
      if (u >= units) continue;
      const int bl = u >> 3, h = (u >> 2) & 1, c = u & 3;
      PlaneUnit wu[RPW];
#pragma unroll
      for (int r = 0; r < RPW; ++r)
        wu[r] = P::decode(P::load(&wl[wave][r][off[r] + bl * P::Bytes], h, c), h, c);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float qf[RPW][8];
#pragma unroll
        for (int r = 0; r < RPW; ++r)
#pragma unroll
          for (int e = 0; e < 8; ++e) qf[r][e] = sbyte_f32(wu[r].q[j][e >> 2], e & 3);
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          if (i >= mrows) break;
          const float* p = &xs[i][256 * bl + 128 * h + 32 * j + 8 * c];
          const float4 a = *reinterpret_cast<const float4*>(p);
          const float4 b = *reinterpret_cast<const float4*>(p + 4);
          const float xv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
          for (int r = 0; r < RPW; ++r) {
            float dot = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) dot = fmaf(qf[r][e], xv[e], dot);
            acc[i][r] = fmaf(wu[r].dsc[j], dot, acc[i][r]);
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
    for (int e = 0; e < 8; ++e) v[e] = u.dsc[j] * sbyte_f32(u.q[j][e >> 2], e & 3);
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
// ------------------------------------------------------------ prefill GEMM
// Y = X W^T with X bf16 [m, k], fp32 Y, on v_mfma_f32_32x32x16_bf16: the
// tile kernel of the Q4_K path (128 weight rows per tile, K steps of 64
// weights, the step's weight tile dequantized to bf16 in a double-buffered LDS
// tile, X fragments straight from global memory, split K with fp32 atomics
// when the tile grid is small), with a plane-format tile fill.  Fill thread
// (row t / 2, half f = t % 2) of step s (part s' = s % 4 of super-block s / 4)
// decodes the 32 weights 64 s' + 32 f + l (l = 0..31) of its row, i.e. h = s'/2,
// j = 2 (s' % 2) + f: one 32-byte low-bit field and one 32-byte high-bit field
// (aligned dwords plus a byte shift, as in the GEMV), two sub-block scales
// and d; each weight (d sc) (q - OFF) rounded once to fp32, then to bf16.
constexpr int kPBN = 128;      // weight rows per tile
constexpr int kPBK = 64;       // weights per K step
constexpr int kPLds = 72;      // bf16 per LDS row: 64 + 8 pad

// A tile-fill thread's share of a 64-k step: the 32 weights l = 0..31 of
// group j of half h (ND = 8 dwords per field), or the 16 weights l = 16 part
// + (0..15) (ND = 4).
template <int FMT, int ND = 8>
struct PlaneFill {
  uint32_t lo[ND + 1], hi[ND + 1];  // low-bit field (ql / qs), high-bit field (qh / hmask)
  uint32_t sc[4];                   // the scale bytes of the half (Q6_K: 8) or all 12 (Q3_K)
  uint32_t d, s;
};

template <int FMT, int ND = 8>
__device__ __forceinline__ void plane_fill_load(const uint8_t* blk, int sp, int f, int part,
                                                PlaneFill<FMT, ND>& r) {
  const int h = sp >> 1, j = 2 * (sp & 1) + f;
  const int lb = ND == 8 ? 0 : 16 * part;
  r.s = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(blk) & 3u);
  if constexpr (FMT == 6) {
    load_field<ND>(blk + 64 * h + 32 * (j & 1) + lb, r.s, r.lo);
    load_field<ND>(blk + 128 + 32 * h + lb, r.s, r.hi);
    uint32_t t[3];
    load_field<2>(blk + 192 + 8 * h, r.s, t);
    r.sc[0] = t[0]; r.sc[1] = t[1]; r.sc[2] = t[2]; r.sc[3] = 0u;
    r.d = *reinterpret_cast<const uint16_t*>(blk + 208);
  } else {
    load_field<ND>(blk + 32 + 32 * h + lb, r.s, r.lo);
    load_field<ND>(blk + lb, r.s, r.hi);
    load_field<3>(blk + 96, r.s, r.sc);
    r.d = *reinterpret_cast<const uint16_t*>(blk + 108);
  }
}

// The thread's bf16 weights as pairs: 32 (l = 0..31 of group j of half h)
// into out[16], or 16 (l = 16 part + (0..15)) into out[8].
template <int FMT, int ND = 8>
__device__ __forceinline__ void plane_fill_decode(const PlaneFill<FMT, ND>& r, int sp, int f,
                                                  int part, uint32_t (&out)[2 * ND]) {
  const int h = sp >> 1, j = 2 * (sp & 1) + f;
  constexpr int NCB = ND / 4;  // sub-blocks of 16 weights the thread covers
  uint32_t L[ND], H[ND];
  align_field<ND>(r.lo, r.s, L);
  align_field<ND>(r.hi, r.s, H);
  const float d = half_bits_to_float(r.d);
  float dsc[NCB];
  if constexpr (FMT == 6) {
    uint32_t S[2];
    align_field<2>(*reinterpret_cast<const uint32_t(*)[3]>(r.sc), r.s, S);
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      const int b = 2 * j + (ND == 8 ? c : part);  // sub-block 8h + 2j + l / 16
      dsc[c] = d * static_cast<float>(static_cast<int8_t>(((b < 4 ? S[0] : S[1]) >> (8 * (b & 3))) & 0xFFu));
    }
  } else {
    uint32_t S[3];
    align_field<3>(r.sc, r.s, S);
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
      const int b = 2 * j + (ND == 8 ? c : part);
      const uint32_t low4 = ((b < 4 ? S[0] : S[1]) >> (8 * (b & 3) + 4 * h)) & 15u;
      const uint32_t top2 = (S[2] >> (8 * (b & 3) + 2 * (2 * h + (j >> 1)))) & 3u;
      dsc[c] = d * static_cast<float>(static_cast<int>(low4 | (top2 << 4)) - 32);
    }
  }
  // Per dword: the low bits shifted to bits 0.. of each byte, the high bits
  // rotated to their place above them (the bits a rotation carries across
  // bytes are masked off), merged with one AND-OR.  Q6_K: low nibble at
  // shift 4 (j / 2), high bits 2j, 2j + 1 to bits 4, 5 (rotate right by
  // 2j - 4); Q3_K: bits 2j, 2j + 1 to 0, 1, hmask bit 4h + j to bit 2.
  const uint32_t lshift = FMT == 6 ? 4u * static_cast<uint32_t>(j >> 1) : 2u * static_cast<uint32_t>(j);
  const uint32_t hrot = FMT == 6 ? static_cast<uint32_t>(2 * j + 28) & 31u
                                 : static_cast<uint32_t>(4 * h + j + 30) & 31u;
  constexpr uint32_t lmask = FMT == 6 ? 0x0F0F0F0Fu : 0x03030303u;
  constexpr uint32_t hmask = FMT == 6 ? 0x30303030u : 0x04040404u;
  // (d sc) (q - OFF) = fma(d sc, q, -(d sc) OFF): OFF is a power of two, so
  // (d sc) OFF is exact and the FMA rounds the exact weight once, as the
  // subtract-then-multiply form does.  Q3_K's quants (0..7) are widened two
  // at a time as fp8 bytes (q 2^-9 exactly), with 2^9 folded into d sc.
  const float off = Planes<FMT>::Off;
  float svs[NCB], nbs[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) {
    nbs[c] = -(dsc[c] * off);
    svs[c] = FMT == 3 ? dsc[c] * kNibbleUnscale : dsc[c];
  }
#pragma unroll
  for (int e = 0; e < ND; ++e) {  // dword e: weights 4e .. 4e + 3 of the thread's run
    const uint32_t q = ((L[e] >> lshift) & lmask) | (__builtin_amdgcn_alignbit(H[e], H[e], hrot) & hmask);
    const float sv = svs[e >> 2], nb = nbs[e >> 2];
    f2_t q01, q23;
    if constexpr (FMT == 3) {
      q01 = fp8x2_lo(q);
      q23 = fp8x2_hi(q);
    } else {
      q01 = f2_t{ubyte_f32(q, 0), ubyte_f32(q, 1)};
      q23 = f2_t{ubyte_f32(q, 2), ubyte_f32(q, 3)};
    }
    out[2 * e] = pack_bf16x2(__builtin_fmaf(sv, q01.x, nb), __builtin_fmaf(sv, q01.y, nb));
    out[2 * e + 1] = pack_bf16x2(__builtin_fmaf(sv, q23.x, nb), __builtin_fmaf(sv, q23.y, nb));
  }
}

template <int FMT, int WAVES_M, int WAVES_N, int TI, int TJ>
__global__ __launch_bounds__(256, 2) void k_gemm_planes(const uint8_t* __restrict__ w,
                                                        const uint16_t* __restrict__ x,
                                                        float* __restrict__ y, int m, int n, int k,
                                                        int steps_per_split, int atomic_out) {
  static_assert(WAVES_M * WAVES_N == 4, "four waves per workgroup");
  static_assert(WAVES_N * 32 * TJ == kPBN, "the tile fill covers 128 weight rows");
  constexpr int BM = WAVES_M * 32 * TI;
  constexpr int BB = Planes<FMT>::Bytes;
  __shared__ __attribute__((aligned(16))) uint16_t ws[2][kPBN * kPLds];
  typedef float f16v_t __attribute__((ext_vector_type(16)));
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int half = lane >> 5;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * kPBN;
  const int nb = k >> 8;
  const int steps = k / kPBK;
  const int s_begin = blockIdx.z * steps_per_split;
  const int s_end = min(steps, s_begin + steps_per_split);
  if (s_begin >= s_end) return;  // uniform over the workgroup, before any barrier

  const int f_row = t >> 1, f_hh = t & 1;
  const uint8_t* f_base = w + static_cast<size_t>(min(n0 + f_row, n - 1)) * nb * BB;
  const uint16_t* a_ptr[TI];
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const int row = min(m0 + wm * 32 * TI + 32 * i + (lane & 31), m - 1);
    a_ptr[i] = x + static_cast<size_t>(row) * k + 32 * half;
  }
  f16v_t acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Loads past the last step re-read the last step (results unused).
  auto load_w = [&](int s, PlaneFill<FMT>& r) {
    const int sc = min(s, s_end - 1);
    plane_fill_load<FMT>(f_base + static_cast<size_t>(sc >> 2) * BB, sc & 3, f_hh, 0, r);
  };
  auto load_x = [&](int s, uint4 (&xr)[TI][4]) {
    const int sc = min(s, s_end - 1);
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const uint16_t* p = a_ptr[i] + static_cast<size_t>(sc) * kPBK;
#pragma unroll
      for (int c = 0; c < 4; ++c) xr[i][c] = *reinterpret_cast<const uint4*>(p + 8 * c);
    }
  };
  auto store_w = [&](int buf, int s, const PlaneFill<FMT>& r) {
    uint32_t v[16];
    plane_fill_decode<FMT>(r, s & 3, f_hh, 0, v);
    uint16_t* dst = &ws[buf][f_row * kPLds + 32 * f_hh];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<uint4*>(dst + 8 * q) = make_uint4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  };
  auto mfma_step = [&](int buf, const uint4 (&xr)[TI][4]) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8_t bfr[TJ];
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int nrow = wn * 32 * TJ + 32 * j + (lane & 31);
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(&ws[buf][nrow * kPLds + 32 * half + 8 * kk]);
      }
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const bf16x8_t afr = __builtin_bit_cast(bf16x8_t, xr[i][kk]);
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr, bfr[j], acc[i][j], 0, 0, 0);
      }
    }
  };

  // The Q4_K tile kernel's pipeline: at step s the MFMAs read LDS buffer s % 2
  // and X registers set s % 2 while the weights of step s + 1 are decoded into
  // the other buffer and step s + 2's X fragments and raw weights are fetched.
  uint4 xA[TI][4], xB[TI][4];
  PlaneFill<FMT> wA, wB;
  load_w(s_begin, wA);
  load_x(s_begin, xA);
  load_x(s_begin + 1, xB);
  store_w(0, s_begin, wA);
  load_w(s_begin + 1, wB);
  load_w(s_begin + 2, wA);
  __syncthreads();
  for (int s = s_begin; s < s_end; s += 2) {
    mfma_step(0, xA);
    load_x(s + 2, xA);
    if (s + 1 < s_end) store_w(1, s + 1, wB);
    load_w(s + 3, wB);
    __syncthreads();
    if (s + 1 >= s_end) break;
    mfma_step(1, xB);
    load_x(s + 3, xB);
    if (s + 2 < s_end) store_w(0, s + 2, wA);
    load_w(s + 4, wA);
    __syncthreads();
  }

  // Accumulator r of a 32x32 tile holds row 8*(r/4) + 4*half + r%4, column lane%32.
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int col = n0 + wn * 32 * TJ + 32 * j + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 32 * TI + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
        if (row < m && col < n) {
          float* dst = y + static_cast<size_t>(row) * n + col;
          if (atomic_out)
            unsafeAtomicAdd(dst, acc[i][j][r]);
          else
            *dst = acc[i][j][r];
        }
      }
    }
}

// Zero fill for split-K outputs (a kernel, not a memset node, so that a
// captured graph replays it faithfully).
__global__ __launch_bounds__(256) void k_zero_planes(float* __restrict__ y, size_t count) {
  const size_t i = (static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i + 4 <= count) {
    *reinterpret_cast<f4_t*>(y + i) = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
  } else {
    for (size_t e = i; e < count; ++e) y[e] = 0.0f;
  }
}

// ------------------------------------------------- GEMM, operands staged in LDS
// The tile kernel above issues, per thread and 64-k step, about 22 dword
// loads of its row's fields and 4 X loads that touch each 128-byte line of
// X twice: counters at m = 512, n = k = 4096 (Q6_K) show the texture
// addresser busy 67% of the time and 0.09 L2 requests per clock per CU,
// i.e. the launch is bound by its memory instructions.  Here both operands
// reach LDS by direct 16-byte copies, and the tile fill reads its fields
// from LDS:
//   * X: per 64-k step the tile's 128 rows x 128 bytes (16 copies, 2 per
//     wave) into a 3-slot ring, two steps ahead, rows XOR-swizzled by 16-byte
//     chunk (lds_copy.h) so a fragment read is conflict-free.
//   * weights: per super-block each of the 128 rows' record as the U 16-byte
//     units from the 16-byte boundary at or below its start (Q6_K: 14, Q3_K:
//     8), into a 2-slot ring, copied at the last step of the super-block
//     before the one that needs it.  Unit u of row r lands at LDS unit
//     PITCH r + u of the slot (PITCH = U + 1, odd, so the rows a wave's fill
//     reads at once fall in different banks; with PITCH = U the 128-byte
//     rows of Q3_K all but shared their banks: 79 against 51 us at m = 512,
//     n = k = 4096 with four waves), so a record keeps its address mod 16
//     and its fields are read as in global memory.  Every wave issues the
//     same number of copies; the pad unit of each row and the lanes past the
//     last row re-read a unit of the matrix into LDS that no fill reads.  A
//     unit past the 16-byte boundary at or above the record's end re-reads
//     the one before it, so no copy leaves the matrix, whose byte size must
//     be a multiple of 16 (the launcher checks).
//   * eight waves, two per SIMD, so that one wave's fill arithmetic and LDS
//     waits run beside the other's MFMAs: the fill (thread t: row t / 4, the
//     16 weights 16 (t % 4) .. +15 of the step) decodes step s + 1 into the
//     other bf16 tile during step s, with the arithmetic above, and wave w
//     runs step s's MFMAs for rows 32 (w % 4) .. +31 and columns
//     64 (w / 4) .. +63 (four waves, one per SIMD, each filling 32 weights
//     and running all 128 columns: 10% slower).
//   * where the time goes (m = 512, n = k = 4096, Q6_K, 51 us; timing-only
//     copies of the kernel): the copies and barriers alone with the zero
//     fill and the split-K atomics take 34 us, of which the atomics about 8
//     and the zero fill 5.6; the fill adds about 12 us and the MFMAs about
//     10, with little overlap (separate copy-only waves did not change it).
//   * waits: at the end of step s the copies of X(s + 1) (issued at step
//     s - 1) and everything before them have landed; the weight copies of a
//     super-block are older than the X copies of the step before its first
//     fill, so one count per phase covers both.
template <int FMT>
struct PlaneStage {
  static constexpr int BB = Planes<FMT>::Bytes;
  static constexpr int U = FMT == 6 ? 14 : 8;  // 16-byte units per row and super-block
  static constexpr int PITCH = U + 1;          // LDS units per row
  static constexpr int Waves = 8, Threads = 64 * Waves;
  static constexpr int WC = (kPBN * PITCH + 64 * Waves - 1) / (64 * Waves);  // weight copies per wave per super-block
  static constexpr int XC = kPBN * 128 / 1024 / Waves;  // X copies per wave per step
  static constexpr int XSlots = 3, WSlots = 2;
  static constexpr int XSlot = kPBN * 128;
  static constexpr int WSlot = WC * Waves * 1024;  // every copy's 1 KiB, the rows' PITCH units first
  static constexpr int TOff = XSlots * XSlot + WSlots * WSlot;
  static constexpr int TSlot = kPBN * kPLds * 2;
  static constexpr int Lds = TOff + 2 * TSlot;
  static_assert((BB + 14 + 15) / 16 <= U, "U units cover a record at any 16-byte offset");
  static_assert(WC * Waves * 64 >= kPBN * PITCH, "the weight copies of a super-block cover the tile");
  static_assert(XC * Waves * 1024 == kPBN * 128, "the X copies of a step cover the tile");
  static_assert(Lds <= 160 * 1024, "LDS budget of one workgroup");
};

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int FMT>
__global__ __launch_bounds__(512, 1) void k_gemm_planes_lds(const uint8_t* __restrict__ w,
                                                            const uint16_t* __restrict__ x,
                                                            float* __restrict__ y, int m, int n,
                                                            int k, int sb_per_split,
                                                            int atomic_out) {
  using P = PlaneStage<FMT>;
  typedef float f16v_t __attribute__((ext_vector_type(16)));
  __shared__ __attribute__((aligned(1024))) uint8_t smem[P::Lds];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int half = lane >> 5;
  const int c32 = lane & 31;
  const int m0 = blockIdx.y * 128, n0 = blockIdx.x * kPBN;
  const int nb = k >> 8;
  const int sb0 = blockIdx.z * sb_per_split;
  const int nsb = min(nb, sb0 + sb_per_split) - sb0;
  if (nsb <= 0) return;  // uniform over the workgroup, before any barrier
  const int nst = 4 * nsb;
  const size_t row_bytes = static_cast<size_t>(nb) * P::BB;

  // X copy q of this wave: tile rows 8 (XC wave + q) .. +7, lane -> (row lane
  // / 8, LDS chunk lane % 8) holding global chunk (lane % 8) ^ swz(row).  Rows
  // past m re-read row m - 1 (not stored).
  const uint16_t* xsrc[P::XC];
#pragma unroll
  for (int q = 0; q < P::XC; ++q) {
    const int row = 8 * (P::XC * wave + q) + (lane >> 3);
    xsrc[q] = x + static_cast<size_t>(min(m0 + row, m - 1)) * k + 256 * static_cast<size_t>(sb0) +
              8 * ((lane & 7) ^ swz(row));
  }
  // Weight copy i of this wave: LDS unit Ui = 64 (WC wave + i) + lane of the
  // slot = unit Ui % PITCH of tile row Ui / PITCH (rows past n re-read row
  // n - 1; the pad unit and the rows past the tile re-read a unit of a
  // record, clamped below).
  const uint8_t* wsrc[P::WC];
  uint32_t wunit[P::WC];
#pragma unroll
  for (int i = 0; i < P::WC; ++i) {
    const int ui = 64 * (P::WC * wave + i) + lane;
    const int r = ui / P::PITCH;
    wunit[i] = static_cast<uint32_t>(ui - r * P::PITCH);
    wsrc[i] = w + static_cast<size_t>(min(n0 + r, n - 1)) * row_bytes +
              static_cast<size_t>(sb0) * P::BB;
  }
  const uint32_t lds0 = lds_address(smem);
  // Steps and super-blocks past the end re-read the last one (into slots no
  // later step reads).
  auto copy_x = [&](int s) {
    const int sc = min(s, nst - 1);
    const uint32_t slot = lds0 + (s % P::XSlots) * P::XSlot;
#pragma unroll
    for (int q = 0; q < P::XC; ++q)
      copy16_to_lds(xsrc[q] + static_cast<size_t>(sc) * kPBK,
                    __builtin_amdgcn_readfirstlane(slot + (P::XC * wave + q) * 1024));
  };
  auto copy_w = [&](int S) {
    const int sc = min(S, nsb - 1);
    const uint32_t slot = lds0 + P::XSlots * P::XSlot + (S % P::WSlots) * P::WSlot;
#pragma unroll
    for (int i = 0; i < P::WC; ++i) {
      const uintptr_t rec = reinterpret_cast<uintptr_t>(wsrc[i]) + static_cast<uintptr_t>(sc) * P::BB;
      const uintptr_t last = ((rec + P::BB + 15) & ~static_cast<uintptr_t>(15)) - 16;
      uintptr_t a = (rec & ~static_cast<uintptr_t>(15)) + 16 * wunit[i];
      a = a < last ? a : last;
      copy16_to_lds(reinterpret_cast<const void*>(a),
                    __builtin_amdgcn_readfirstlane(slot + (P::WC * wave + i) * 1024));
    }
  };

  // Fill thread: row t / 4, weights 32 f_hh + 16 part + (0..15) of a step.
  const int f_row = t >> 2, f_hh = (t >> 1) & 1, part = t & 1;
  const uint32_t f_mis = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>(w + static_cast<size_t>(min(n0 + f_row, n - 1)) * row_bytes +
                                  static_cast<size_t>(sb0) * P::BB) & 15u);
  auto fill = [&](int s) {
    const int S = s >> 2, sp = s & 3;
    const uint32_t off = (f_mis + static_cast<uint32_t>(S * P::BB)) & 15u;
    const uint8_t* blk = smem + P::XSlots * P::XSlot + (S % P::WSlots) * P::WSlot +
                         f_row * (P::PITCH * 16) + off;
    PlaneFill<FMT, 4> r;
    plane_fill_load<FMT, 4>(blk, sp, f_hh, part, r);
    uint32_t v[8];
    plane_fill_decode<FMT, 4>(r, sp, f_hh, part, v);
    uint16_t* dst = reinterpret_cast<uint16_t*>(smem + P::TOff + (s & 1) * P::TSlot) +
                    f_row * kPLds + 32 * f_hh + 16 * part;
#pragma unroll
    for (int q = 0; q < 2; ++q)
      *reinterpret_cast<uint4*>(dst + 8 * q) =
          make_uint4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
  };

  const int wm = wave & 3, wn = wave >> 2;
  f16v_t acc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
  // Wave: tile rows 32 wm .. +31, columns 64 wn .. +63.  Lane half h takes
  // k = 32 h + 8 kk + (0..7) of the step in slice kk, for X and weights alike.
  auto mfma_step = [&](int s) {
    const uint8_t* xb = smem + (s % P::XSlots) * P::XSlot;
    const uint16_t* tb = reinterpret_cast<const uint16_t*>(smem + P::TOff + (s & 1) * P::TSlot);
    const int xr = 32 * wm + c32;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bf16x8_t a =
          *reinterpret_cast<const bf16x8_t*>(xb + xr * 128 + (((4 * half + kk) ^ swz(xr)) << 4));
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bf16x8_t b = *reinterpret_cast<const bf16x8_t*>(
            tb + (64 * wn + 32 * j + c32) * kPLds + 32 * half + 8 * kk);
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
      }
    }
  };

  // Prologue: W(0), X(0), X(1), W(1); W(0) and X(0) land; step 0 is filled.
  copy_w(0);
  copy_x(0);
  copy_x(1);
  copy_w(1);
  wait_copies_barrier<P::XC + P::WC>();
  fill(0);
  lds_barrier();
  // Step s (phase p = s % 4 of its super-block): X(s + 2) into the slot of
  // step s - 1, at phase 3 the weights of super-block S + 2 into the slot of
  // S; fill step s + 1; MFMAs of step s.  Younger than X(s + 1) at the end:
  // this step's X copies, and the weight copies of a phase-3 step (this one
  // at p = 3, the one before at p = 0).
  auto step = [&](int s, int p) {
    copy_x(s + 2);
    if (p == 3) copy_w((s >> 2) + 2);
    if (s + 1 < nst) fill(s + 1);
    mfma_step(s);
    if (p == 0 || p == 3)
      wait_copies_barrier<P::XC + P::WC>();
    else
      wait_copies_barrier<P::XC>();
  };
  for (int s = 0; s < nst; s += 4) {
    step(s, 0);
    step(s + 1, 1);
    step(s + 2, 2);
    step(s + 3, 3);
  }
  wait_copies<0>();  // the re-read copies past the end land before the LDS is released

  // Accumulator r of a 32x32 tile holds row 8 (r / 4) + 4 half + r % 4, column lane % 32.
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = n0 + 64 * wn + 32 * j + c32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = m0 + 32 * wm + 8 * (r >> 2) + 4 * half + (r & 3);
      if (row < m && col < n) {
        float* dst = y + static_cast<size_t>(row) * n + col;
        if (atomic_out)
          unsafeAtomicAdd(dst, acc[j][r]);
        else
          *dst = acc[j][r];
      }
    }
  }
}

template <int FMT>
hipError_t launch_gemm_planes_staged(const uint8_t* w, const uint16_t* x, float* y, int m, int n,
                                     int k, hipStream_t stream) {
  const int tiles_m = (m + 127) / 128, tiles_n = (n + kPBN - 1) / kPBN;
  const int nb = k / 256;
  // Split K (whole super-blocks) until the grid reaches one workgroup per CU.
  int splits = 1;
  while (tiles_m * tiles_n * splits * 2 <= 256 && splits * 2 <= nb / 2) splits *= 2;
  const int per = (nb + splits - 1) / splits;
  splits = (nb + per - 1) / per;
  if (splits > 1) {
    const size_t count = static_cast<size_t>(m) * n;
    hipLaunchKernelGGL(k_zero_planes, dim3(static_cast<unsigned>((count / 4 + 256) / 256)), dim3(256),
                       0, stream, y, count);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k_gemm_planes_lds<FMT>), dim3(tiles_n, tiles_m, splits),
                     dim3(PlaneStage<FMT>::Threads), 0,
                     stream, w, x, y, m, n, k, per, splits > 1 ? 1 : 0);
  return hipGetLastError();
}

template <int FMT, int WAVES_M, int WAVES_N, int TI, int TJ>
hipError_t launch_gemm_planes_tiles(const uint8_t* w, const uint16_t* x, float* y, int m, int n,
                                    int k, hipStream_t stream) {
  constexpr int BM = WAVES_M * 32 * TI;
  const int tiles_m = (m + BM - 1) / BM, tiles_n = (n + kPBN - 1) / kPBN;
  const int steps = k / kPBK;
  // Split K until the grid reaches one workgroup per CU (256 on MI355X).
  int splits = 1;
  while (tiles_m * tiles_n * splits * 2 <= 256 && splits * 2 <= steps / 8) splits *= 2;
  const int per = (steps + splits - 1) / splits;
  splits = (steps + per - 1) / per;
  if (splits > 1) {
    const size_t count = static_cast<size_t>(m) * n;
    hipLaunchKernelGGL(k_zero_planes, dim3(static_cast<unsigned>((count / 4 + 256) / 256)), dim3(256),
                       0, stream, y, count);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k_gemm_planes<FMT, WAVES_M, WAVES_N, TI, TJ>), dim3(tiles_n, tiles_m, splits),
                     dim3(256), 0, stream, w, x, y, m, n, k, per, splits > 1 ? 1 : 0);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_gemm_planes(const uint8_t* w, const uint16_t* x, float* y, int64_t m, int64_t n,
                              int64_t k, hipStream_t stream) {
  const int mi = static_cast<int>(m), ni = static_cast<int>(n), ki = static_cast<int>(k);
  if (mi <= 32) return launch_gemm_planes_tiles<FMT, 1, 4, 1, 1>(w, x, y, mi, ni, ki, stream);
  // The staged kernel's weight copies round each record out to 16-byte
  // boundaries, which stay inside the matrix when its byte size is a
  // multiple of 16.
  if ((n * (k / 256) * Planes<FMT>::Bytes) % 16 == 0)
    return launch_gemm_planes_staged<FMT>(w, x, y, mi, ni, ki, stream);
  return launch_gemm_planes_tiles<FMT, 4, 1, 1, 4>(w, x, y, mi, ni, ki, stream);
}

// One pass of up to MT x rows: the LDS-staged kernel when the copies'
// 16-byte rounding stays inside the matrix, else the direct one.
template <int FMT, int WAVES, int RPW, int MT>
hipError_t launch_gemv_planes_pass(const uint8_t* w, const float* x, float* y, int n, int k,
                                   int mm, bool staged, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>((n + WAVES * RPW - 1) / (WAVES * RPW)));
  if (staged)
    hipLaunchKernelGGL((k_gemv_planes_lds<FMT, WAVES, RPW, MT>), grid, dim3(64 * WAVES), 0, stream,
                       w, x, y, n, k, mm);
  else
    hipLaunchKernelGGL((k_gemv_planes<FMT, WAVES, RPW, MT>), grid, dim3(64 * WAVES), 0, stream, w,
                       x, y, n, k, mm);
  return hipGetLastError();
}

// Batch 1: one row per wave, kPlaneDecodeWaves waves per workgroup.  Passes of
// 2 to 4 x rows: two rows per wave, 8 waves (each unit widened once serves
// both rows' dots for every x row).
template <int FMT>
hipError_t launch_gemv_planes(const uint8_t* w, const float* x, float* y, int64_t m, int64_t n,
                              int64_t k, hipStream_t stream) {
  const int ni = static_cast<int>(n), ki = static_cast<int>(k);
  const bool staged = (n * (k / 256)) % 8 == 0;
  for (int64_t i0 = 0; i0 < m; i0 += 4) {
    const int mm = static_cast<int>(m - i0 < 4 ? m - i0 : 4);
    const float* xs = x + i0 * k;
    float* ys = y + i0 * n;
    hipError_t e;
    if (mm == 1)
      e = launch_gemv_planes_pass<FMT, kPlaneDecodeWaves, 1, 1>(w, xs, ys, ni, ki, mm, staged,
                                                                stream);
    else if (mm == 2)
      e = launch_gemv_planes_pass<FMT, 8, 2, 2>(w, xs, ys, ni, ki, mm, staged, stream);
    else
      e = launch_gemv_planes_pass<FMT, 8, 2, 4>(w, xs, ys, ni, ki, mm, staged, stream);
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

hipError_t launch_q6k_gemm(const uint8_t* w, const uint16_t* x, float* y, int64_t m, int64_t n,
                           int64_t k, hipStream_t stream) {
  return launch_gemm_planes<6>(w, x, y, m, n, k, stream);
}
hipError_t launch_q3k_gemm(const uint8_t* w, const uint16_t* x, float* y, int64_t m, int64_t n,
                           int64_t k, hipStream_t stream) {
  return launch_gemm_planes<3>(w, x, y, m, n, k, stream);
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
