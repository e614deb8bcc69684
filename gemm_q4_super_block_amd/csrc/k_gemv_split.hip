// k_gemv_split.hip -- Q4_K and Q5_K GEMV for batches of 5 to 32 rows on bf16 MFMA.
//
// What it computes is q4k_gemv's y = x W^T (fp32 x, fp32 y, the same
// tolerance, 1e-4 * sum|w x| per output).  At these batch sizes one fp32 FMA
// per weight per batch row is more VALU work than the weight stream can hide,
// so the products go to the matrix cores, as the daScript PR page's tile
// kernels do for batches ("CPU kernel parity ...": token reuse in the tile
// kernels), with fp32-GEMV accuracy kept by splitting both operands.
//
// Design for gfx950:
//   * v_mfma_f32_16x16x32_bf16: one MFMA covers 32 weights (K) of 16 weight
//     rows (N) for 16 batch rows (M).
//   * every weight is formed exactly first, w = fma(d sc, q, -dmin m) (the
//     dequant export's bits), then split w = w_hi + w_lo with w_hi = bf16(w)
//     and w_lo = bf16(w - w_hi); x likewise (x_hi, x_lo).  Three MFMAs per
//     tile, w_hi x_hi + w_hi x_lo + w_lo x_hi, leave out w_lo x_lo and the two
//     residuals, each at most 2^-16 |w x| (bf16 keeps 8 significant bits), so
//     every product is within 3 * 2^-16 of w x, and every partial product is
//     exact in the fp32 accumulator.  A weight that is zero contributes
//     exactly zero: a block whose weights cancel (d sc q = dmin m) gives +-0,
//     which applying the scales to separate sums of q x and x cannot.
//   * operand layout (both operands alike, so any internal k order gives the
//     same contraction): lane l supplies row l % 16 (a batch row of x, or a
//     weight row) and the 8 consecutive k of its k-group l / 16.  For quant
//     group g a lane's 8 quant bytes (32g + 8 (l/16) ..) hold the low nibbles
//     of sub-block 2g and the high nibbles of sub-block 2g + 1.  The result
//     tile holds batch row 4 (l/16) + r, weight row l % 16 in register r.
//   * a workgroup of 4 waves owns 16 NT weight rows (NT = 2 from 8192 rows);
//     wave w takes super-blocks w, w + 4, ... of the rows (prefetching the
//     next one's header and quants), and the four partial tiles are summed
//     through LDS at the end.
#include <hip/hip_runtime.h>

#include "lds_copy.h"
#include "q4k_device.h"
#include "q4k_launch.h"

namespace q4k {
namespace {

typedef float f4v_t __attribute__((ext_vector_type(4)));

// 8 fp32 values -> (hi, lo) bf16x8 with hi = bf16(v), lo = bf16(v - hi).
__device__ __forceinline__ void split_bf16(const float (&v)[8], bf16x8_t& hi, bf16x8_t& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
    const float r0 = v[2 * i] - __builtin_bit_cast(float, h[i] << 16);
    const float r1 = v[2 * i + 1] - __builtin_bit_cast(float, h[i] & 0xFFFF0000u);
    l[i] = pack_bf16x2(r0, r1);
  }
  hi = __builtin_bit_cast(bf16x8_t, uint4{h[0], h[1], h[2], h[3]});
  lo = __builtin_bit_cast(bf16x8_t, uint4{l[0], l[1], l[2], l[3]});
}

// The 8 exact weights of 8 quant bytes' low (HIGH = false) or high nibbles,
// in byte order: fma(a, q * 2^-9, -b) on the fp8-widened nibbles (Q4_K, a =
// d sc 2^9) or fma(a, q, -b) on exactly widened 5-bit quants (Q5_K, a = d sc,
// fifth bits from bit `bit` of the 8 high-bit bytes h).
template <bool HIGH, int FMT>
__device__ __forceinline__ void weights8(uint2 q, uint2 h, int bit, float a, float b,
                                         float (&w)[8]) {
  uint32_t u0 = HIGH ? (q.x >> 4) & 0x0F0F0F0Fu : q.x & 0x0F0F0F0Fu;
  uint32_t u1 = HIGH ? (q.y >> 4) & 0x0F0F0F0Fu : q.y & 0x0F0F0F0Fu;
  if constexpr (FMT == 5) {
    u0 |= ((h.x >> bit) & 0x01010101u) << 4;
    u1 |= ((h.y >> bit) & 0x01010101u) << 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w[e] = __builtin_fmaf(a, ubyte_f32(u0, e), -b);
      w[4 + e] = __builtin_fmaf(a, ubyte_f32(u1, e), -b);
    }
  } else {
    const f2_t p0 = fp8x2_lo(u0), p1 = fp8x2_hi(u0), p2 = fp8x2_lo(u1), p3 = fp8x2_hi(u1);
    w[0] = __builtin_fmaf(a, p0.x, -b);
    w[1] = __builtin_fmaf(a, p0.y, -b);
    w[2] = __builtin_fmaf(a, p1.x, -b);
    w[3] = __builtin_fmaf(a, p1.y, -b);
    w[4] = __builtin_fmaf(a, p2.x, -b);
    w[5] = __builtin_fmaf(a, p2.y, -b);
    w[6] = __builtin_fmaf(a, p3.x, -b);
    w[7] = __builtin_fmaf(a, p3.y, -b);
  }
}

// STAGED: a wave's super-blocks of the 16 NT weight rows reach LDS by direct
// copies (each row's record contiguous, in a wave-private two-slot ring one
// super-block ahead) and the lanes read their header and quant bytes from
// there.  Loaded straight from memory instead, each load instruction touches
// 16 rows' 16 or 32 bytes, one record (row_bytes) apart.
template <int MT, int NT, int WV, int FMT, bool STAGED>
__global__ __launch_bounds__(64 * WV) void k_gemv_split(const uint8_t* __restrict__ w,
                                                        const float* __restrict__ x,
                                                        float* __restrict__ y, int m, int n,
                                                        int k) {
  constexpr int BB = block_bytes<FMT>();
  constexpr int WUnits = 16 * NT * BB / 16;  // 16-byte units of one super-block of the rows
  constexpr int WC = (WUnits + 63) / 64;     // copies of them per wave
  constexpr int WSlot = WUnits * 16;
  constexpr int RedBytes = WV * MT * NT * 4 * 64 * 4;
  constexpr int RingBytes = STAGED ? WV * 2 * WSlot : 0;
  constexpr int SmemBytes = RingBytes > RedBytes ? RingBytes : RedBytes;
  static_assert(SmemBytes <= 160 * 1024, "LDS budget of one workgroup");
  static_assert(WC + 16 * MT <= 63, "vmcnt range");
  // The weight rings, and after the K loop the partial tiles (over them).
  __shared__ __attribute__((aligned(1024))) uint8_t smem[SmemBytes];
  auto red = reinterpret_cast<float (*)[MT][NT][4][64]>(smem);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nl = lane & 15, kg = lane >> 4;
  const int nb = k >> 8;
  const int n0 = blockIdx.x * 16 * NT;

  // Weight rows of this lane (clamped; rows past n are computed, not stored).
  const uint8_t* wrow[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
    wrow[t] = w + static_cast<size_t>(min(n0 + 16 * t + nl, n - 1)) * nb * block_bytes<FMT>();
  // Batch rows this lane feeds as the A operand; rows past m read row m - 1 and
  // are zeroed.
  const float* xrow[MT];
  bool xvalid[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    xrow[t] = x + static_cast<size_t>(min(16 * t + nl, m - 1)) * k;
    xvalid[t] = 16 * t + nl < m;
  }

  f4v_t acc[MT][NT];
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[a][b] = f4v_t{0.0f, 0.0f, 0.0f, 0.0f};

  // Q5_K: the 8 high-bit bytes qh[8 kg ..] of the lane's k serve all four
  // groups (bit 2g for the low nibbles, 2g + 1 for the high ones).
  constexpr int kQOff = FMT == 5 ? kQ5QuantOffset : 16;
  struct WBlock {
    uint4 hd[NT];
    uint2 q[NT][4];
    uint2 qh[NT];
  };
  auto load_w = [&](int b, WBlock& wb) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint8_t* p = wrow[t] + static_cast<size_t>(b) * block_bytes<FMT>();
      wb.hd[t] = *reinterpret_cast<const uint4*>(p);
#pragma unroll
      for (int g = 0; g < 4; ++g)
        wb.q[t][g] = *reinterpret_cast<const uint2*>(p + kQOff + 32 * g + 8 * kg);
      if constexpr (FMT == 5) wb.qh[t] = *reinterpret_cast<const uint2*>(p + kQ5HighOffset + 8 * kg);
    }
  };

  // Staged: copy i of a super-block fills units min(64 i, WUnits - 64) + lane
  // of the slot, unit U = part U % (BB / 16) of row U / (BB / 16) (rows past n
  // read row n - 1; the last copy repeats some units of the one before, with
  // the same data and place).
  const uint32_t row_bytes = static_cast<uint32_t>(nb) * BB;
  const uint8_t* const wt = w + static_cast<size_t>(n0) * row_bytes;
  uint32_t woff[STAGED ? WC : 1];
  if constexpr (STAGED) {
#pragma unroll
    for (int i = 0; i < WC; ++i) {
      const int U = min(64 * i, WUnits - 64) + lane;
      const int r = U / (BB / 16);
      woff[i] = static_cast<uint32_t>(min(r, n - 1 - n0)) * row_bytes + (U - r * (BB / 16)) * 16;
    }
  }
  uint8_t* const ring = smem + (STAGED ? wave * 2 * WSlot : 0);
  auto copy_w = [&](int b, int slot) {
    const uint8_t* base = wt + static_cast<size_t>(min(b, nb - 1)) * BB;
    const uint32_t dst = lds_address(ring) + slot * WSlot;
#pragma unroll
    for (int i = 0; i < WC; ++i) copy16_to_lds_so(woff[i], base, dst + min(64 * i, WUnits - 64) * 16);
  };
  auto read_w = [&](int slot, WBlock& wb) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const uint8_t* p = ring + slot * WSlot + (16 * t + nl) * BB;
      wb.hd[t] = *reinterpret_cast<const uint4*>(p);
#pragma unroll
      for (int g = 0; g < 4; ++g)
        wb.q[t][g] = *reinterpret_cast<const uint2*>(p + kQOff + 32 * g + 8 * kg);
      if constexpr (FMT == 5) wb.qh[t] = *reinterpret_cast<const uint2*>(p + kQ5HighOffset + 8 * kg);
    }
  };

  WBlock cur, nxt;
  int b = wave;
  int slot = 0;
  if constexpr (STAGED) {
    if (b < nb) copy_w(b, 0);
  } else {
    if (b < nb) load_w(b, cur);
  }
  for (; b < nb; b += WV, slot ^= 1) {
    // Staged: the next super-block's copies (past the end the last one again,
    // so every pass issues the same number) ahead of this one's x loads.
    if constexpr (STAGED) {
      copy_w(b + WV, slot ^ 1);
    } else {
      if (b + WV < nb) load_w(b + WV, nxt);
    }
    // x of the whole super-block, this lane's 8 k of each of its 8 sub-blocks:
    // issued together so that one L2 round trip serves the four quant groups.
    float4 xr[MT][8][2];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int sb = 0; sb < 8; ++sb) {
        const float* p = xrow[t] + 256 * b + 32 * sb + 8 * kg;
        xr[t][sb][0] = *reinterpret_cast<const float4*>(p);
        xr[t][sb][1] = *reinterpret_cast<const float4*>(p + 4);
      }
    if constexpr (STAGED) {
      // Issued after this super-block's copies: the next copies and the x loads.
      wait_copies<WC + 16 * MT>();
      read_w(slot, cur);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      // x of sub-blocks 2g (s = 0) and 2g + 1 (s = 1), split into bf16 hi + lo
      bf16x8_t ahi[MT][2], alo[MT][2];
#pragma unroll
      for (int t = 0; t < MT; ++t) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const float4 u = xr[t][2 * g + s][0];
          const float4 v = xr[t][2 * g + s][1];
          float xv[8] = {u.x, u.y, u.z, u.w, v.x, v.y, v.z, v.w};
          if (!xvalid[t]) {
#pragma unroll
            for (int e = 0; e < 8; ++e) xv[e] = 0.0f;
          }
          split_bf16(xv, ahi[t][s], alo[t][s]);
        }
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        GroupScales sc = group_scales(cur.hd[nt], g);
        if constexpr (FMT == 5) {  // exact 5-bit quants: the scale is d sc, without 2^9
          sc.a_lo *= 1.0f / kNibbleUnscale;
          sc.a_hi *= 1.0f / kNibbleUnscale;
        }
        float wl[8], wh[8];
        weights8<false, FMT>(cur.q[nt][g], cur.qh[nt], 2 * g, sc.a_lo, sc.b_lo, wl);
        weights8<true, FMT>(cur.q[nt][g], cur.qh[nt], 2 * g + 1, sc.a_hi, sc.b_hi, wh);
        bf16x8_t wl_hi, wl_lo, wh_hi, wh_lo;
        split_bf16(wl, wl_hi, wl_lo);
        split_bf16(wh, wh_hi, wh_lo);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          f4v_t d = acc[t][nt];
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[t][0], wl_hi, d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[t][0], wl_hi, d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[t][0], wl_lo, d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[t][1], wh_hi, d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[t][1], wh_hi, d, 0, 0, 0);
          d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[t][1], wh_lo, d, 0, 0, 0);
          acc[t][nt] = d;
        }
      }
    }
    if constexpr (!STAGED) cur = nxt;
  }
  (void)slot;
  if constexpr (STAGED) wait_copies<0>();
  __syncthreads();  // every wave is done with its ring before the tiles go over it

  // Sum the waves' partial tiles: wave v finishes the (t, nt) tiles with
  // (t * NT + nt) % WV == v and stores them.  Tile register r holds batch row
  // 4 kg + r, weight row nl.
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][t][nt][r][lane] = acc[t][nt][r];
  __syncthreads();
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if ((t * NT + nt) % WV != wave) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = red[0][t][nt][r][lane];
#pragma unroll
        for (int src = 1; src < WV; ++src) v += red[src][t][nt][r][lane];
        const int row = 16 * t + 4 * kg + r, col = n0 + 16 * nt + nl;
        if (row < m && col < n) y[static_cast<size_t>(row) * n + col] = v;
      }
    }
}

}  // namespace

bool gemv_split_supported(int64_t m) { return m >= kGemvSplitMinM && m <= 32; }

namespace {

// One 16-row batch tile for m <= 16, two above.  A workgroup owns 16 NT
// weight rows and its WV waves split K (wave v takes super-blocks v, v + WV,
// ...), so each x split serves NT weight tiles.  Matrices of at least
// kSplitTallRows rows take 64-row tiles on 8 waves (224 workgroups at 14336
// rows); smaller ones 16-row tiles on 8 waves (256 at 4096 rows), so that
// the grid still covers the CUs.
constexpr int kSplitTallRows = 8192;
constexpr bool kSplitStaged = true;

template <int MT, int NT, int WV, int FMT>
void launch_split_tiles(const uint8_t* w, const float* x, float* y, int m, int n, int k,
                        hipStream_t stream) {
  // Q4_K's 64-row tiles stage their weights through LDS (Q5_K's 176-byte
  // records would need 176 KiB of rings; the 16-row tiles of two batch tiles
  // run out of registers).
  constexpr bool kStaged = FMT == 4 && NT == 4 && kSplitStaged;
  hipLaunchKernelGGL((k_gemv_split<MT, NT, WV, FMT, kStaged>), dim3((n + 16 * NT - 1) / (16 * NT)),
                     dim3(64 * WV), 0, stream, w, x, y, m, n, k);
}

template <int FMT>
hipError_t launch_split_fmt(const uint8_t* w, const float* x, float* y, int64_t m, int64_t n,
                            int64_t k, hipStream_t stream) {
  const int mi = static_cast<int>(m), ni = static_cast<int>(n), ki = static_cast<int>(k);
  if (ni >= kSplitTallRows) {
    if (mi <= 16)
      launch_split_tiles<1, 4, 8, FMT>(w, x, y, mi, ni, ki, stream);
    else
      launch_split_tiles<2, 4, 8, FMT>(w, x, y, mi, ni, ki, stream);
  } else {
    if (mi <= 16)
      launch_split_tiles<1, 1, 8, FMT>(w, x, y, mi, ni, ki, stream);
    else
      launch_split_tiles<2, 1, 8, FMT>(w, x, y, mi, ni, ki, stream);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_split(const uint8_t* w, const float* x, float* y, int64_t m, int64_t n,
                             int64_t k, hipStream_t stream) {
  return launch_split_fmt<4>(w, x, y, m, n, k, stream);
}

hipError_t launch_q5k_gemv_split(const uint8_t* w, const float* x, float* y, int64_t m, int64_t n,
                                 int64_t k, hipStream_t stream) {
  return launch_split_fmt<5>(w, x, y, m, n, k, stream);
}

}  // namespace q4k
