// k_gemm_stream.hip -- Q4_K and Q5_K GEMM for batches of at most 32 rows (bf16 X).
//
// What it computes is q4k_gemm's (q5k_gemm's) Y = X W^T (fp32 accumulate,
// the same per-weight dequantization as the prefill tiles).  With 32 rows or fewer the
// work is a weight stream: every weight is used by at most 32 products, and a
// launch is as fast as the weight bytes reach the CUs and get dequantized.
// The K-slice tiles share one LDS ring among the four waves of a workgroup
// and keep them in step with a barrier per 64-wide K step; this kernel lets
// each wave stream on its own.
//
// Design for gfx950:
//   * a workgroup owns 32 NB weight rows and the batch rows; its four waves
//     split K by super-block (wave v takes super-blocks v, v + 4, ...), and
//     sum their partial tiles through LDS once, at the end.
//   * each wave copies only what it reads, into its own part of LDS, with
//     direct global -> LDS copies: its super-block of the workgroup's rows
//     (32 NB records of 144 or 176 bytes, contiguous per row) into a 2-slot
//     ring one super-block ahead, and the 64-wide K step of the first XR batch
//     rows of X that each quant group needs (XR rows x 128 bytes, XOR-swizzled
//     rows) into a 5-slot ring four steps ahead (Q5_K with XR >= 16: 4 slots,
//     three ahead).  A wave waits only for its own
//     copies (s_waitcnt vmcnt): no barrier until the partial tiles are summed.
//     The copies take a scalar base and a fixed per-lane 32-bit offset, so
//     the stream costs no vector instructions beyond the copies themselves.
//   * XR = 8 or 16 rows (m <= 16): 32-row weight tiles (NB = 1), two
//     workgroups per CU (at most 78 KiB of LDS each); XR = 32: 64-row tiles
//     (NB = 2), one workgroup per CU.
//   * v_mfma_f32_32x32x16_bf16 with X as A (batch rows) and W as B (weight
//     rows).  Lane (c, h) = (lane % 32, lane / 32) of quant group g reads the
//     16 quant bytes 16 h .. 16 h + 15 of weight row c and the X chunks of the
//     same k: MFMA (p, u) takes the nibbles p (0 low, 1 high) of bytes
//     16 h + 8 u .. +7, k = 64 g + 32 p + 16 h + 8 u + (0..7) in both operands
//     (any k order gives the same contraction, as long as both use it).
//     A rows at or past XR repeat row XR - 1; their outputs are not stored.
//   * weights as in the other GEMM kernels: fma(d sc 2^9, q 2^-9, -dmin m)
//     (Q5_K: fma(d sc, q, -dmin m) on the exactly widened 5-bit quant), one
//     rounding, then bf16; a cancelling block gives exact zeros.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "lds_copy.h"
#include "q4k_device.h"
#include "q4k_launch.h"

namespace q4k {
namespace {

typedef float f16x_t __attribute__((ext_vector_type(16)));

template <int NB, int XR, int FMT>
struct Stream {
  static constexpr int BB = block_bytes<FMT>();       // 144 (Q4_K) or 176 (Q5_K)
  static constexpr int Units = BB / 16;              // 16-byte units per record
  static constexpr int RW = 32 * NB;                 // weight rows per workgroup
  static constexpr int WUnits = RW * Units;          // 16-byte units of one super-block of them
  static constexpr int WC = (WUnits + 63) / 64;      // weight copies per super-block
  static constexpr int WSlot = WUnits * 16;
  static constexpr int WSlots = 2;
  static constexpr int XSlot = XR * 128;             // XR batch rows x 64 k of bf16
  static constexpr int XC = XR / 8;                  // X copies per step (8 rows each)
  // X issued XSlots - 1 steps ahead (Q5_K's larger records leave room for one
  // step less at 16 and 32 rows).
  static constexpr int XSlots = FMT == 5 && XR >= 16 ? 4 : 5;
  static constexpr int XOff = WSlots * WSlot;
  static constexpr int WaveLds = XOff + XSlots * XSlot;
  static constexpr int Lds = 4 * WaveLds;
  static constexpr int MinBlocks = NB == 1 ? 2 : 1;  // workgroups per CU
  static_assert(Lds * MinBlocks <= 160 * 1024, "LDS budget of the workgroups of one CU");
  static_assert(NB * 4 * 1024 <= WaveLds, "a wave's partial tile fits its own LDS part");
  // W(t + 1) is issued at step 4 t, before X(4 t + XSlots - 1): waiting for
  // X(i + 1) covers the weights step i + 1 reads.
  static_assert(XSlots + 3 <= 4 * WSlots, "weight ring depth");
  // Copies issued after X(i + 1) when step i (group g) waits for it: the X
  // copies of XSlots - 2 later steps, and a weight super-block when one of
  // those steps starts a super-block (g < XSlots - 2).
  static constexpr int wait_count(int g) { return (XSlots - 2) * XC + (g < XSlots - 2 ? WC : 0); }
  static_assert((XSlots - 2) * XC + WC <= 63, "vmcnt range");
};

// Sub-block scales of one super-block header: a = d sc 2^9 (Q5_K: d sc),
// b = dmin m for sub-blocks 0..7.
struct SbScales {
  float a[8], b[8];
};

template <int FMT>
__device__ __forceinline__ void sb_scales(const uint4 h, SbScales& s) {
  const uint32_t sc_lo = h.y & 0x3F3F3F3Fu;
  const uint32_t mn_lo = h.z & 0x3F3F3F3Fu;
  const uint32_t sc_hi = (h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u);
  const uint32_t mn_hi = ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u);
  // Q4_K nibbles are widened as fp8 (q 2^-9); Q5_K quants exactly.
  const float d = half_bits_to_float(h.x & 0xFFFFu) * (FMT == 5 ? 1.0f : kNibbleUnscale);
  const float dmin = half_bits_to_float(h.x >> 16);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    s.a[e] = d * ubyte_f32(sc_lo, e);
    s.a[4 + e] = d * ubyte_f32(sc_hi, e);
    s.b[e] = dmin * ubyte_f32(mn_lo, e);
    s.b[4 + e] = dmin * ubyte_f32(mn_hi, e);
  }
}

template <int NB, int XR, int FMT>
__global__ __launch_bounds__(256, NB == 1 ? 2 : 1) void k_gemm_q4k_stream(const uint8_t* __restrict__ w,
                                                            const uint16_t* __restrict__ x,
                                                            float* __restrict__ y, int m, int n,
                                                            int k) {
  using C = Stream<NB, XR, FMT>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::Lds];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 31;
  const int h = lane >> 5;
  const int nsb = k >> 8;
  const int n0 = blockIdx.x * C::RW;
  // This wave's super-blocks: wave, wave + 4, ...; cnt of them, 4 cnt steps.
  const int cnt = nsb > wave ? (nsb - wave + 3) >> 2 : 0;
  const int steps = 4 * cnt;
  const uint32_t row_bytes = static_cast<uint32_t>(nsb) * C::BB;
  // The tile's first weight row, in 64 bits; offsets inside its 32 NB rows
  // stay below 2^32 (k <= 2^24, checked by the C ABI).
  const uint8_t* const wt = w + static_cast<size_t>(n0) * row_bytes;
  uint8_t* const mine = smem + wave * C::WaveLds;
  const uint32_t lds_mine = lds_address(mine);

  // Weight copy i: units min(64 i, WUnits - 64) + lane of the slot, unit U =
  // part U % Units of row U / Units (the last copy repeats some units of the
  // one before, with the same data and place).  Rows past n read row n - 1.
  uint32_t woff[C::WC];
#pragma unroll
  for (int i = 0; i < C::WC; ++i) {
    const int U = min(64 * i, C::WUnits - 64) + lane;
    const int r = U / C::Units;
    woff[i] = static_cast<uint32_t>(min(r, n - 1 - n0)) * row_bytes + (U - r * C::Units) * 16;
  }
  // X copy q fills slot rows 8 q .. 8 q + 7; lane -> (row, LDS chunk lane % 8)
  // holding X chunk (lane % 8) ^ swz(row).  Rows past m read row m - 1 (their
  // outputs are not stored).
  uint32_t xoff[C::XC];
#pragma unroll
  for (int q = 0; q < C::XC; ++q) {
    const int row = 8 * q + (lane >> 3);
    xoff[q] = (static_cast<uint32_t>(min(row, m - 1)) * static_cast<uint32_t>(k) +
               8 * ((lane & 7) ^ swz(row))) * 2;
  }
  // Super-block of this wave's t-th step group (indices past the end repeat the last).
  auto sb_of = [&](int t) { return wave + 4 * min(t, cnt - 1); };
  auto copy_w = [&](int t) {
    const uint8_t* base = wt + static_cast<size_t>(sb_of(t)) * C::BB;
    const uint32_t dst = lds_mine + (t & 1) * C::WSlot;
#pragma unroll
    for (int i = 0; i < C::WC; ++i)
      copy16_to_lds_so(woff[i], base, dst + min(64 * i, C::WUnits - 64) * 16);
  };
  auto copy_x = [&](int i) {
    const int ic = min(i, steps - 1);
    const size_t k0 = static_cast<size_t>(sb_of(ic >> 2)) * 256 + 64 * (ic & 3);
    const uint16_t* base = x + k0;
    const uint32_t dst = lds_mine + C::XOff + (i % C::XSlots) * C::XSlot;
#pragma unroll
    for (int q = 0; q < C::XC; ++q) copy16_to_lds_so(xoff[q], base, dst + q * 1024);
  };

  // Fragments of one step: the quant bytes of group g of each weight row
  // block (Q5_K: and the high-bit bytes of the same positions, bit 2 g + p of
  // each holding the fifth bit), and the four X chunks of batch row c.
  constexpr int kQOff = FMT == 5 ? kQ5QuantOffset : 16;
  struct Frag {
    uint4 q[NB];
    uint4 qh[FMT == 5 ? NB : 1];
    bf16x8_t xa[4];  // [2 p + u]
  };
  auto read_frag = [&](int i, Frag& f) {
    const uint8_t* ws = mine + ((i >> 2) & 1) * C::WSlot;
    const int g = i & 3;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const uint8_t* rec = ws + (32 * j + c) * C::BB;
      f.q[j] = *reinterpret_cast<const uint4*>(rec + kQOff + 32 * g + 16 * h);
      if constexpr (FMT == 5) f.qh[j] = *reinterpret_cast<const uint4*>(rec + kQ5HighOffset + 16 * h);
    }
    const int xr = min(c, XR - 1);
    const uint8_t* xs = mine + C::XOff + (i % C::XSlots) * C::XSlot + xr * 128;
#pragma unroll
    for (int pu = 0; pu < 4; ++pu) {
      const int ch = 4 * (pu >> 1) + 2 * h + (pu & 1);
      f.xa[pu] = *reinterpret_cast<const bf16x8_t*>(xs + ((ch ^ swz(xr)) << 4));
    }
  };
  auto read_hdr = [&](int t, uint4 (&hd)[NB]) {
    const uint8_t* ws = mine + (t & 1) * C::WSlot;
#pragma unroll
    for (int j = 0; j < NB; ++j)
      hd[j] = *reinterpret_cast<const uint4*>(ws + (32 * j + c) * C::BB);
  };

  f16x_t acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;

  if (cnt > 0) {
    // Prologue: W(0), X(0..3); X(0) (and W(0) before it) landed.
    copy_w(0);
#pragma unroll
    for (int i = 0; i < C::XSlots - 1; ++i) copy_x(i);
    wait_copies<(C::XSlots - 2) * C::XC>();
    Frag fa, fb;
    uint4 hd[NB];
    SbScales sc[NB];
    read_hdr(0, hd);
    read_frag(0, fa);
#pragma unroll
    for (int j = 0; j < NB; ++j) sb_scales<FMT>(hd[j], sc[j]);

    // Step i (group g of super-block t): issue W(t + 1) at g = 0 and X(i + 4);
    // dequantize and multiply step i from fc; wait for X(i + 1) (and with it
    // W(t + 1)); read step i + 1's fragments into fn (and at g = 3 the next
    // super-block's headers, decoded at the top of the next step).
    auto step = [&](int i, auto gc, Frag& fc, Frag& fn) {
      constexpr int g = decltype(gc)::value;
      if (g == 0) copy_w((i >> 2) + 1);
      copy_x(i + C::XSlots - 1);
      if (g == 0 && i > 0) {
#pragma unroll
        for (int j = 0; j < NB; ++j) sb_scales<FMT>(hd[j], sc[j]);
      }
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            const uint32_t d0 = u ? fc.q[j].z : fc.q[j].x, d1 = u ? fc.q[j].w : fc.q[j].y;
            bf16x8_t b;
            if constexpr (FMT == 5) {
              const uint32_t h0 = u ? fc.qh[j].z : fc.qh[j].x, h1 = u ? fc.qh[j].w : fc.qh[j].y;
              b = __builtin_bit_cast(
                  bf16x8_t, dequant8_bf16_q5(q5_bytes(d0, h0, 4 * p, 2 * g + p),
                                             q5_bytes(d1, h1, 4 * p, 2 * g + p),
                                             sc[j].a[2 * g + p], sc[j].b[2 * g + p]));
            } else {
              b = dequant8_bf16(d0, d1, 4 * p, sc[j].a[2 * g + p], sc[j].b[2 * g + p]);
            }
            acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fc.xa[2 * p + u], b, acc[j], 0, 0, 0);
          }
      __builtin_amdgcn_sched_barrier(0);
      wait_copies<C::wait_count(g)>();
      __builtin_amdgcn_sched_barrier(0);
      read_frag(i + 1, fn);
      if (g == 3) read_hdr((i >> 2) + 1, hd);
    };
    for (int i = 0; i < steps; i += 4) {
      step(i, std::integral_constant<int, 0>{}, fa, fb);
      step(i + 1, std::integral_constant<int, 1>{}, fb, fa);
      step(i + 2, std::integral_constant<int, 2>{}, fa, fb);
      step(i + 3, std::integral_constant<int, 3>{}, fb, fa);
    }
    // Every copy of this wave has landed before its LDS part is reused.
    wait_copies<0>();
  }

  // Sum the four waves' partial tiles: wave v writes accumulator r4 (4
  // registers) of block j as 1-KiB unit 4 j + r4 of its own LDS part, then
  // finishes units v NB .. v NB + NB - 1 from all four parts.
  uint8_t* const out = mine;
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      *reinterpret_cast<f4_t*>(out + (4 * j + r4) * 1024 + lane * 16) =
          f4_t{acc[j][4 * r4], acc[j][4 * r4 + 1], acc[j][4 * r4 + 2], acc[j][4 * r4 + 3]};
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
  for (int uu = 0; uu < NB; ++uu) {
    const int u = wave * NB + uu;
    const int j = u >> 2, r4 = u & 3;
    f4_t v = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int src = 0; src < 4; ++src)
      v += *reinterpret_cast<const f4_t*>(smem + src * C::WaveLds + u * 1024 + lane * 16);
    // Accumulator r of a 32x32 tile holds batch row 8 (r / 4) + 4 h + r % 4,
    // weight row lane % 32.
    const int col = n0 + 32 * j + c;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 8 * r4 + 4 * h + e;
      if (row < m && col < n) y[static_cast<size_t>(row) * n + col] = v[e];
    }
  }
}

}  // namespace

int gemm_stream_tiles(int64_t n) { return static_cast<int>((n + 63) / 64); }

template <int FMT>
hipError_t launch_stream(const uint8_t* w, const uint16_t* x, float* y, int64_t m, int64_t n,
                         int64_t k, hipStream_t stream) {
  const int mi = static_cast<int>(m), ni = static_cast<int>(n), ki = static_cast<int>(k);
  if (mi <= 8) {
    hipLaunchKernelGGL((k_gemm_q4k_stream<1, 8, FMT>), dim3((ni + 31) / 32), dim3(256), 0,
                       stream, w, x, y, mi, ni, ki);
  } else if (mi <= 16) {
    hipLaunchKernelGGL((k_gemm_q4k_stream<1, 16, FMT>), dim3((ni + 31) / 32), dim3(256), 0,
                       stream, w, x, y, mi, ni, ki);
  } else {
    hipLaunchKernelGGL((k_gemm_q4k_stream<2, 32, FMT>), dim3((ni + 63) / 64), dim3(256), 0,
                       stream, w, x, y, mi, ni, ki);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_stream(const uint8_t* w, const uint16_t* x, float* y, int64_t m, int64_t n,
                              int64_t k, hipStream_t stream) {
  return launch_stream<4>(w, x, y, m, n, k, stream);
}

hipError_t launch_q5k_gemm_stream(const uint8_t* w, const uint16_t* x, float* y, int64_t m,
                                  int64_t n, int64_t k, hipStream_t stream) {
  return launch_stream<5>(w, x, y, m, n, k, stream);
}

}  // namespace q4k
