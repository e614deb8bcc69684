// k_gemv.hip -- decode GEMV on Q4_K weights, and the gate/up SwiGLU stage.
//
// y[i, r] = sum_c W[r, c] x[i, c] for a few activation rows i (decode: one).
// The dequantization is fused into an fp32 FMA dot product ("Writing an
// ESIMD Fused Kernel From Reverse-Engineered Assembly", "Getting Q4_K Right":
// dequant feeding a dot with a SIMD reduce), and the gate and up projections
// of the MLP share one read of x with h = silu(g) * u formed in registers
// ("Building ESIMD Infrastructure": MUL_MAT + MUL_MAT + SWIGLU).
//
// Work mapping (wave64):
//   * lane = 4*b + g: b = 0..15 is a super-block slot, g = 0..3 a quant group.
//     One K step covers 16 consecutive super-blocks of a row (4096 weights); a
//     lane reads the block header (16 B) and the 32 quant bytes of its group
//     (two 16-byte loads) -- weights 64g..64g+63 of the block: 32 low nibbles
//     of sub-block 2g and 32 high nibbles of 2g+1.  A wave's load covers one
//     row's 2304 contiguous bytes, which streams HBM as well as a flat copy.
//   * a wave owns a set of R consecutive rows (2R with the gate/up pair) and
//     reuses each staged x value for all of them; waves are persistent: each
//     walks row sets with a stride of the whole grid, and the (row set, K step)
//     items are pipelined -- the next item's weights are in flight while the
//     current one is computed (two register sets, the loop unrolled by two).
//   * x (MT activation rows, a chunk of K at a time) is staged once per
//     workgroup in LDS, skewed by 16 bytes every 256 so that the lanes of a
//     wave -- whose 64-float slices start 256 bytes apart -- hit distinct
//     banks.
//   * every weight is formed exactly before it meets x: fma(a_j, q_l, -b_j)
//     rounds d sc q - dmin m once, the same bits as the dequant export, and
//     the dot is then a plain fp32 FMA chain over exact weights.  (Applying
//     the scales per sub-block, a_j sum q x - b_j sum x, is one FMA per weight
//     cheaper but loses the result when a_j q ~ b_j: a block whose weights
//     cancel to zero would return the rounding noise of two large sums.)
//   * quants are widened with v_cvt_pk_f32_fp8 (a masked nibble byte is the
//     fp8 value q * 2^-9), two per instruction, and each weight is formed once
//     whatever MT.
//   * lanes reduce with DPP and two cross-row swizzles; lane 0 stores.
//   * batch 1 with k <= 16384 -- the GEMV at any row count, and the gate/up
//     pair of the MLP -- takes k_gemv_decode: the same per-lane
//     arithmetic with one row per wave, every K step's weights issued at once
//     and x staged by direct global -> LDS copies.  The gate and up rows of a
//     row index go to two waves of one workgroup, which read the one staged x;
//     the gate wave forms h from u passed through LDS.
#include <hip/hip_runtime.h>

#include <atomic>

#include "lds_copy.h"
#include "q4k_device.h"
#include "q4k_launch.h"

namespace q4k {
namespace {

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

__device__ __forceinline__ float silu(float t) { return t / (1.0f + expf(-t)); }

// Elements of K staged per pass: MT rows of x share roughly 64 KiB of LDS.
// Always a multiple of one K step (4096 elements).
template <int MT>
constexpr int kXChunk = MT == 1 ? 16384 : MT == 2 ? 8192 : 4096;

__device__ __forceinline__ int xs_index(int i) { return i + ((i >> 6) << 2); }

// Floats of LDS per staged activation row (x skewed by 16 bytes every 256).
__host__ __device__ constexpr int xs_stride(int kc) { return kc + kc / 16; }

__host__ __device__ constexpr size_t gemv_lds_bytes(int mt, int kc) {
  return static_cast<size_t>(mt) * xs_stride(kc) * sizeof(float);
}

template <int R, int NW, int FMT>
struct WRegs {
  uint4 hd[NW][R], qa[NW][R], qb[NW][R];
  uint4 h0[NW][FMT == 5 ? R : 1], h1[NW][FMT == 5 ? R : 1];  // Q5_K high bits
};

// MT activation rows per pass, R weight rows per wave (times NW = 2 weight
// matrices for the gate/up pair), NWV waves per workgroup.  FMT: 4 (Q4_K) or
// 5 (Q5_K: a lane also loads
// the block's 32 high-bit bytes and widens its 5-bit quant bytes exactly with
// v_cvt_f32_ubyte, so its scale is d*sc without the 2^9 of the fp8 path).
template <int MT, int R, bool GLU, int NWV, int FMT>
__device__ __forceinline__ void gemv_body(const uint8_t* __restrict__ w,
                                          const uint8_t* __restrict__ w2,
                                          const float* __restrict__ x, float* __restrict__ y,
                                          int m, int n, int k) {
  static_assert(!GLU || MT == 1, "the gate/up pair runs at batch 1");
  constexpr int NW = GLU ? 2 : 1;
  constexpr int NT = 64 * NWV;
  extern __shared__ float smem[];
  const int kc_max = min(k, kXChunk<MT>);
  const int xst = xs_stride(kc_max);
  float* xs = smem;  // [MT][xst]
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int b = lane >> 2;
  const int g = lane & 3;
  const int kb_count = k >> 8;
  constexpr int kBB = block_bytes<FMT>();
  constexpr int kQOff = FMT == 5 ? kQ5QuantOffset : 16;
  const size_t row_bytes = static_cast<size_t>(kb_count) * kBB;
  const int nsets = (n + R - 1) / R;
  const int gw = blockIdx.x * NWV + wave;
  const int tw = gridDim.x * NWV;
  const int my_sets = gw < nsets ? (nsets - 1 - gw) / tw + 1 : 0;
  // With at most one row set per wave the accumulators stay in registers
  // across K chunks (the gate/up pair needs the full dot before silu);
  // otherwise each chunk's partial dot is added into y.
  const bool single = tw >= nsets;

  float acc[NW][R][MT];
#pragma unroll
  for (int u = 0; u < NW; ++u)
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int i = 0; i < MT; ++i) acc[u][r][i] = 0.0f;

  for (int c0 = 0; c0 < k; c0 += kXChunk<MT>) {
    const int kc = min(kXChunk<MT>, k - c0);
    const int s_begin = c0 >> 12;
    const int ns = (kc + 4095) >> 12;  // K steps in this chunk
    const int jobs = my_sets * ns;
    const bool last_chunk = c0 + kc >= k;

    auto issue = [&](int j, WRegs<R, NW, FMT>& B) {
      const int si = j / ns;
      const int st = s_begin + (j - si * ns);
      const int row0 = (gw + si * tw) * R;
      const int kb = min(st * 16 + b, kb_count - 1);
#pragma unroll
      for (int u = 0; u < NW; ++u) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int row = min(row0 + r, n - 1);
          const uint8_t* p = (u ? w2 : w) + row * row_bytes + static_cast<size_t>(kb) * kBB;
          B.hd[u][r] = load16(p);
          B.qa[u][r] = load16(p + kQOff + 32 * g);
          B.qb[u][r] = load16(p + kQOff + 16 + 32 * g);
          if constexpr (FMT == 5) {
            B.h0[u][r] = load16(p + kQ5HighOffset);
            B.h1[u][r] = load16(p + kQ5HighOffset + 16);
          }
        }
      }
    };

    auto compute = [&](int j, const WRegs<R, NW, FMT>& B) {
      const int si = j / ns;
      const int sl = j - si * ns;
      const int st = s_begin + sl;
      // Lanes past the last super-block (ragged last step) read block 0 of
      // the chunk and x slot 0 -- valid memory -- and add nothing.
      const bool active = st * 16 + b < kb_count;
      const int kb_local = active ? st * 16 + b - (c0 >> 8) : 0;
      const int xo = xs_index(kb_local * kQK + 64 * g);
      // Scales of the lane's two sub-blocks (2g: low nibbles, 2g+1: high).
      GroupScales sc[NW][R];
#pragma unroll
      for (int u = 0; u < NW; ++u)
#pragma unroll
        for (int r = 0; r < R; ++r) {
          sc[u][r] = group_scales(B.hd[u][r], g);
          if constexpr (FMT == 5) {  // the quants are exact integers, not q * 2^-9
            sc[u][r].a_lo *= 1.0f / kNibbleUnscale;
            sc[u][r].a_hi *= 1.0f / kNibbleUnscale;
          }
        }
      float pl[NW][R][MT], ph[NW][R][MT];
#pragma unroll
      for (int u = 0; u < NW; ++u)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int i = 0; i < MT; ++i) pl[u][r][i] = ph[u][r][i] = 0.0f;
      // At batch 1, x is read one 4-float slice ahead of its use; batches
      // read at use (their many accumulators leave no registers to spare).
      // A scheduling fence per slice keeps the compiler from hoisting all the
      // reads of a step (and spilling).
      constexpr bool kAhead = MT == 1;
      f4_t xl_n[MT], xh_n[MT];
      if constexpr (kAhead) {
        xl_n[0] = *reinterpret_cast<const f4_t*>(xs + xo);
        xh_n[0] = *reinterpret_cast<const f4_t*>(xs + xo + 32);
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        f4_t xl[MT], xh[MT];
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          if constexpr (kAhead) {
            xl[i] = xl_n[i];
            xh[i] = xh_n[i];
            if (c < 7) {
              xl_n[i] = *reinterpret_cast<const f4_t*>(xs + i * xst + xo + 4 * c + 4);
              xh_n[i] = *reinterpret_cast<const f4_t*>(xs + i * xst + xo + 36 + 4 * c);
            }
          } else {
            xl[i] = *reinterpret_cast<const f4_t*>(xs + i * xst + xo + 4 * c);
            xh[i] = *reinterpret_cast<const f4_t*>(xs + i * xst + xo + 32 + 4 * c);
          }
        }
#pragma unroll
        for (int u = 0; u < NW; ++u) {
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const uint32_t v = c < 4 ? word(B.qa[u][r], c) : word(B.qb[u][r], c - 4);
            f2_t l01, l23, h01, h23;
            if constexpr (FMT == 5) {
              // High-bit dword c: qh bytes 4c .. 4c+3, the fifth bits of
              // weights 64g + 4c + i (bit 2g) and 64g + 32 + 4c + i (bit 2g+1).
              const uint32_t hw = c < 4 ? word(B.h0[u][r], c) : word(B.h1[u][r], c - 4);
              const uint32_t lo = q5_bytes(v, hw, 0, 2 * g);
              const uint32_t hi = q5_bytes(v, hw, 4, 2 * g + 1);
              l01 = f2_t{ubyte_f32(lo, 0), ubyte_f32(lo, 1)};
              l23 = f2_t{ubyte_f32(lo, 2), ubyte_f32(lo, 3)};
              h01 = f2_t{ubyte_f32(hi, 0), ubyte_f32(hi, 1)};
              h23 = f2_t{ubyte_f32(hi, 2), ubyte_f32(hi, 3)};
            } else {
              const uint32_t lo = v & 0x0F0F0F0Fu;
              const uint32_t hi = (v >> 4) & 0x0F0F0F0Fu;
              l01 = fp8x2_lo(lo);
              l23 = fp8x2_hi(lo);
              h01 = fp8x2_lo(hi);
              h23 = fp8x2_hi(hi);
            }
            const GroupScales& s = sc[u][r];
            const float wl0 = __builtin_fmaf(s.a_lo, l01.x, -s.b_lo);
            const float wl1 = __builtin_fmaf(s.a_lo, l01.y, -s.b_lo);
            const float wl2 = __builtin_fmaf(s.a_lo, l23.x, -s.b_lo);
            const float wl3 = __builtin_fmaf(s.a_lo, l23.y, -s.b_lo);
            const float wh0 = __builtin_fmaf(s.a_hi, h01.x, -s.b_hi);
            const float wh1 = __builtin_fmaf(s.a_hi, h01.y, -s.b_hi);
            const float wh2 = __builtin_fmaf(s.a_hi, h23.x, -s.b_hi);
            const float wh3 = __builtin_fmaf(s.a_hi, h23.y, -s.b_hi);
#pragma unroll
            for (int i = 0; i < MT; ++i) {
              float a = pl[u][r][i];
              a = __builtin_fmaf(wl0, xl[i].x, a);
              a = __builtin_fmaf(wl1, xl[i].y, a);
              a = __builtin_fmaf(wl2, xl[i].z, a);
              a = __builtin_fmaf(wl3, xl[i].w, a);
              pl[u][r][i] = a;
              float e = ph[u][r][i];
              e = __builtin_fmaf(wh0, xh[i].x, e);
              e = __builtin_fmaf(wh1, xh[i].y, e);
              e = __builtin_fmaf(wh2, xh[i].z, e);
              e = __builtin_fmaf(wh3, xh[i].w, e);
              ph[u][r][i] = e;
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int u = 0; u < NW; ++u)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int i = 0; i < MT; ++i) acc[u][r][i] += active ? pl[u][r][i] + ph[u][r][i] : 0.0f;
      if (sl != ns - 1 || (single && !last_chunk)) return;
      // Row set finished (for this chunk): reduce, store, reset.
      const int row0 = (gw + si * tw) * R;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = row0 + r;
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          float v = wave_sum(acc[0][r][i]);
          if constexpr (GLU) v = silu(v) * wave_sum(acc[NW - 1][r][i]);
          if (lane == 0 && row < n && i < m) {
            float* dst = y + static_cast<size_t>(i) * n + row;
            if (single || c0 == 0) {
              *dst = v;
            } else {
              *dst += v;
            }
          }
#pragma unroll
          for (int u = 0; u < NW; ++u) acc[u][r][i] = 0.0f;
        }
      }
    };

    // x staging, 16 floats per thread and pass.  The first pass's x loads are
    // issued before the first weights: loads complete in order, so x (a few
    // L2 hits) then lands first and the staging barrier does not wait for the
    // weights of every wave of the workgroup.
    auto load_x16 = [&](int idx, f4_t (&v)[4]) {
      const int i = idx / kc;
      const int e = idx - i * kc;
      v[0] = v[1] = v[2] = v[3] = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
      if (i < m) {
        const f4_t* src = reinterpret_cast<const f4_t*>(x + static_cast<size_t>(i) * k + c0 + e);
        v[0] = src[0];
        v[1] = src[1];
        v[2] = src[2];
        v[3] = src[3];
      }
    };
    auto store_x16 = [&](int idx, const f4_t (&v)[4]) {
      const int i = idx / kc;
      const int e = idx - i * kc;
      f4_t* dst = reinterpret_cast<f4_t*>(xs + i * xst + xs_index(e));
      dst[0] = v[0];
      dst[1] = v[1];
      dst[2] = v[2];
      dst[3] = v[3];
    };
    const bool first = 16 * t < MT * kc;
    f4_t v0[4];
    if (first) load_x16(16 * t, v0);
    WRegs<R, NW, FMT> bufA, bufB;
    if (jobs > 0) issue(0, bufA);
    if (c0 > 0) __syncthreads();  // every wave is done with the previous chunk
    if (first) store_x16(16 * t, v0);
    for (int idx = 16 * t + 16 * NT; idx < MT * kc; idx += 16 * NT) {
      f4_t v[4];
      load_x16(idx, v);
      store_x16(idx, v);
    }
    __syncthreads();

    for (int j = 0; j < jobs; j += 2) {
      if (j + 1 < jobs) issue(j + 1, bufB);
      compute(j, bufA);
      if (j + 1 >= jobs) break;
      if (j + 2 < jobs) issue(j + 2, bufA);
      compute(j + 1, bufB);
    }
  }
}

template <int MT, int R, bool GLU, int NWV, int FMT = 4>
__global__ __launch_bounds__(64 * NWV) void k_gemv_q4k(const uint8_t* __restrict__ w,
                                                       const uint8_t* __restrict__ w2,
                                                       const float* __restrict__ x,
                                                       float* __restrict__ y, int m, int n,
                                                       int k) {
  gemv_body<MT, R, GLU, NWV, FMT>(w, w2, x, y, m, n, k);
}

// Batch-1 GEMV for k <= 4096 NS (NS K steps of 4096): the arithmetic of
// gemv_body<1, 1, false, 16> (same
// loads, the same per-lane order of every rounding, step partials added in
// step order, so the results are bit-identical), with the generality a
// single row per wave does not need taken out: no row-set or chunk loops,
// every step's weight loads issued at once, and x staged by direct global ->
// LDS copies (issued before the weight loads) instead of loads and LDS
// stores.  NW waves (rows) per workgroup; 8 measured fastest at 4096 x 4096
// (4.7 us against 4.9 for 4 and 5.0 for 16), two workgroups per CU each
// staging its own copy of x (from L2).  The LDS holds x in 16-byte units with
// one spare unit after every 16 (unit 16 G + r at position 17 G + r, the
// layout xs_index gives the general kernel): the 16 lanes of a quarter-wave
// read units 16 G + c for 16 consecutive G, which fall in 16 different bank
// groups, and a lane's 16 units of a step sit at immediate offsets from one
// address.  The staging copies fill the positions in order, each lane
// fetching the unit its position holds.
//
// GLU: the gate/up pair of the MLP.  Waves 2 i and 2 i + 1 take row i of the
// workgroup in W_gate (w) and W_up (w2), both reading the one staged x, and
// y = h = silu(g) * u from the two dots (u passed through LDS).
//
// FMT 5: Q5_K blocks, with the two 16-byte loads of the high-bit plane per
// step and the quant bytes widened as gemv_body does for that format.
template <int NW, int NS, bool GLU, int FMT>
__global__ __launch_bounds__(64 * NW) void k_gemv_decode(const uint8_t* __restrict__ w,
                                                         const uint8_t* __restrict__ w2,
                                                         const float* __restrict__ x,
                                                         float* __restrict__ y, int n, int k) {
  constexpr int XPOS = 17 * 64 * NS;  // LDS positions: 17 per 16 x units
  constexpr int RW = GLU ? NW / 2 : NW;  // rows per workgroup
  __shared__ __attribute__((aligned(1024))) float xs[4 * XPOS];
  __shared__ float up[GLU ? RW : 1];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int b = lane >> 2;
  const int g = lane & 3;
  const int nsb = k >> 8;
  const int row = blockIdx.x * RW + (GLU ? wave >> 1 : wave);
  const bool is_up = GLU && (wave & 1);
  // x: copy q of this wave fills positions 64 (wave + NW q) .. + 63, lane l
  // position p = 17 grp + r, r = p mod 17 (kept as the copies advance by
  // 64 NW positions); spare positions and units past k / 4 take the last unit
  // of their group or of x (never read).
  {
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    int grp = (64 * wave + lane) / 17;
    int r = 64 * wave + lane - 17 * grp;
#pragma unroll
    for (int q = 0; q < (XPOS + 64 * NW - 1) / (64 * NW); ++q) {
      const int base = 64 * (wu + NW * q);
      if (base < XPOS) {
        const int u = min(16 * grp + min(r, 15), (k >> 2) - 1);
        copy16_to_lds(x + 4 * u, lds_address(xs) + 16u * static_cast<uint32_t>(base));
      }
      r += (64 * NW) % 17;
      grp += (64 * NW) / 17;
      if (r >= 17) {
        r -= 17;
        ++grp;
      }
    }
  }
  // Weights of this lane, step st: header and the 32 quant bytes of group g
  // of block 16 st + b (lanes past the last block read the last one and add
  // nothing).
  constexpr int kBB = block_bytes<FMT>();
  constexpr int kQOff = FMT == 5 ? kQ5QuantOffset : 16;
  constexpr int kLoads = FMT == 5 ? 5 : 3;  // 16-byte weight loads per step
  const size_t row_bytes = static_cast<size_t>(nsb) * kBB;
  const uint8_t* const wr = (is_up ? w2 : w) + static_cast<size_t>(min(row, n - 1)) * row_bytes;
  uint4 hd[NS], qa[NS], qb[NS], h0[FMT == 5 ? NS : 1], h1[FMT == 5 ? NS : 1];
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    const uint8_t* p = wr + static_cast<size_t>(min(16 * st + b, nsb - 1)) * kBB;
    hd[st] = load16(p);
    qa[st] = load16(p + kQOff + 32 * g);
    qb[st] = load16(p + kQOff + 16 + 32 * g);
    if constexpr (FMT == 5) {
      h0[st] = load16(p + kQ5HighOffset);
      h1[st] = load16(p + kQ5HighOffset + 16);
    }
  }
  // The x copies were issued before the kLoads NS weight loads: they have
  // landed once at most kLoads NS loads are in flight.
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(kLoads * NS) : "memory");

  float acc = 0.0f;
#pragma unroll
  for (int st = 0; st < NS; ++st) {
    const bool active = 16 * st + b < nsb;
    const int kb = active ? 16 * st + b : 0;
    // units 16 (4 kb + g) + c: c < 8 low-nibble weights, c >= 8 high
    const f4_t* xg = reinterpret_cast<const f4_t*>(xs) + 17 * (4 * kb + g);
    GroupScales s = group_scales(hd[st], g);
    if constexpr (FMT == 5) {  // the quants are exact integers, not q * 2^-9
      s.a_lo *= 1.0f / kNibbleUnscale;
      s.a_hi *= 1.0f / kNibbleUnscale;
    }
    float pl = 0.0f, ph = 0.0f;
    f4_t xl_n = xg[0], xh_n = xg[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const f4_t xl = xl_n, xh = xh_n;
      if (c < 7) {
        xl_n = xg[c + 1];
        xh_n = xg[c + 9];
      }
      const uint32_t v = c < 4 ? word(qa[st], c) : word(qb[st], c - 4);
      f2_t l01, l23, h01, h23;
      if constexpr (FMT == 5) {
        const uint32_t hw = c < 4 ? word(h0[st], c) : word(h1[st], c - 4);
        const uint32_t lo = q5_bytes(v, hw, 0, 2 * g);
        const uint32_t hi = q5_bytes(v, hw, 4, 2 * g + 1);
        l01 = f2_t{ubyte_f32(lo, 0), ubyte_f32(lo, 1)};
        l23 = f2_t{ubyte_f32(lo, 2), ubyte_f32(lo, 3)};
        h01 = f2_t{ubyte_f32(hi, 0), ubyte_f32(hi, 1)};
        h23 = f2_t{ubyte_f32(hi, 2), ubyte_f32(hi, 3)};
      } else {
        const uint32_t lo = v & 0x0F0F0F0Fu;
        const uint32_t hi = (v >> 4) & 0x0F0F0F0Fu;
        l01 = fp8x2_lo(lo);
        l23 = fp8x2_hi(lo);
        h01 = fp8x2_lo(hi);
        h23 = fp8x2_hi(hi);
      }
      const float wl0 = __builtin_fmaf(s.a_lo, l01.x, -s.b_lo);
      const float wl1 = __builtin_fmaf(s.a_lo, l01.y, -s.b_lo);
      const float wl2 = __builtin_fmaf(s.a_lo, l23.x, -s.b_lo);
      const float wl3 = __builtin_fmaf(s.a_lo, l23.y, -s.b_lo);
      const float wh0 = __builtin_fmaf(s.a_hi, h01.x, -s.b_hi);
      const float wh1 = __builtin_fmaf(s.a_hi, h01.y, -s.b_hi);
      const float wh2 = __builtin_fmaf(s.a_hi, h23.x, -s.b_hi);
      const float wh3 = __builtin_fmaf(s.a_hi, h23.y, -s.b_hi);
      pl = __builtin_fmaf(wl0, xl.x, pl);
      pl = __builtin_fmaf(wl1, xl.y, pl);
      pl = __builtin_fmaf(wl2, xl.z, pl);
      pl = __builtin_fmaf(wl3, xl.w, pl);
      ph = __builtin_fmaf(wh0, xh.x, ph);
      ph = __builtin_fmaf(wh1, xh.y, ph);
      ph = __builtin_fmaf(wh2, xh.z, ph);
      ph = __builtin_fmaf(wh3, xh.w, ph);
      __builtin_amdgcn_sched_barrier(0);
    }
    acc += active ? pl + ph : 0.0f;
  }
  const float v = wave_sum(acc);
  if constexpr (GLU) {
    if (is_up && lane == 0) up[wave >> 1] = v;
    __syncthreads();
    if (!is_up && lane == 0 && row < n) y[row] = silu(v) * up[wave >> 1];
  } else {
    if (lane == 0 && row < n) y[row] = v;
  }
}

// Independent batch-1 GEMVs of one shape in one persistent launch: y[l] =
// W[l] x[l] for l < layers (k <= kGemvLayersMaxK).  The work mapping of the
// batch-1 GEMV above (lane = super-block slot x quant group, one row per
// wave at a time, 16 waves per workgroup, one workgroup per CU), with the
// (layer, row, K step) items of a wave pipelined across layer boundaries:
// while a wave computes its last row of layer l, the weights of its first row
// of layer l + 1 are in flight, so the weight stream does not stop between
// layers.  x is double-buffered in LDS: x[l + 1] is loaded into registers when
// layer l starts and stored to the other buffer when it ends, then one
// workgroup barrier per layer.  (Staging every layer's x up front, with no
// barrier per layer, measured slower: 32.3 against 30.4 us.)
struct LayerPtrs {
  const uint8_t* w[kGemvMaxLayers];
  const float* x[kGemvMaxLayers];
  float* y[kGemvMaxLayers];
};

constexpr int kLayerWaves = 16;
// LDS of the layered GEMV: two x buffers at the largest k.
constexpr size_t kLayersLdsBytes =
    2 * static_cast<size_t>(xs_stride(kGemvLayersMaxK)) * sizeof(float);

__global__ __launch_bounds__(64 * kLayerWaves) void k_gemv_layers(LayerPtrs p, int layers, int n,
                                                                  int k) {
  constexpr int NT = 64 * kLayerWaves;
  extern __shared__ float smem[];
  const int xst = xs_stride(k);
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int b = lane >> 2;
  const int g = lane & 3;
  const int kb_count = k >> 8;
  const size_t row_bytes = static_cast<size_t>(kb_count) * kBlockBytes;
  const int ns = (k + 4095) >> 12;  // K steps per row
  const int gw = blockIdx.x * kLayerWaves + wave;
  const int tw = gridDim.x * kLayerWaves;
  const int my_rows = gw < n ? (n - 1 - gw) / tw + 1 : 0;
  const int per_layer = my_rows * ns;  // this wave's items per layer
  const int jobs = per_layer * layers;

  auto decode_item = [&](int j, int& l, int& row, int& st) {
    l = j / per_layer;
    const int r = j - l * per_layer;
    const int si = r / ns;
    st = r - si * ns;
    row = gw + si * tw;
  };
  auto issue = [&](int j, WRegs<1, 1, 4>& B) {
    int l, row, st;
    decode_item(j, l, row, st);
    const int kb = min(st * 16 + b, kb_count - 1);
    const uint8_t* q = p.w[l] + row * row_bytes + static_cast<size_t>(kb) * kBlockBytes;
    B.hd[0][0] = load16(q);
    B.qa[0][0] = load16(q + 16 + 32 * g);
    B.qb[0][0] = load16(q + 32 + 32 * g);
  };
  float acc = 0.0f;
  auto compute = [&](int j, const WRegs<1, 1, 4>& B) {
    int l, row, st;
    decode_item(j, l, row, st);
    const float* xs = smem + (l & 1) * xst;
    const bool active = st * 16 + b < kb_count;
    const int xo = xs_index((active ? st * 16 + b : 0) * kQK + 64 * g);
    const GroupScales sc = group_scales(B.hd[0][0], g);
    float pl = 0.0f, ph = 0.0f;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const f4_t xl = *reinterpret_cast<const f4_t*>(xs + xo + 4 * c);
      const f4_t xh = *reinterpret_cast<const f4_t*>(xs + xo + 32 + 4 * c);
      const uint32_t v = c < 4 ? word(B.qa[0][0], c) : word(B.qb[0][0], c - 4);
      const uint32_t lo = v & 0x0F0F0F0Fu;
      const uint32_t hi = (v >> 4) & 0x0F0F0F0Fu;
      const f2_t l01 = fp8x2_lo(lo), l23 = fp8x2_hi(lo), h01 = fp8x2_lo(hi), h23 = fp8x2_hi(hi);
      pl = __builtin_fmaf(__builtin_fmaf(sc.a_lo, l01.x, -sc.b_lo), xl.x, pl);
      pl = __builtin_fmaf(__builtin_fmaf(sc.a_lo, l01.y, -sc.b_lo), xl.y, pl);
      pl = __builtin_fmaf(__builtin_fmaf(sc.a_lo, l23.x, -sc.b_lo), xl.z, pl);
      pl = __builtin_fmaf(__builtin_fmaf(sc.a_lo, l23.y, -sc.b_lo), xl.w, pl);
      ph = __builtin_fmaf(__builtin_fmaf(sc.a_hi, h01.x, -sc.b_hi), xh.x, ph);
      ph = __builtin_fmaf(__builtin_fmaf(sc.a_hi, h01.y, -sc.b_hi), xh.y, ph);
      ph = __builtin_fmaf(__builtin_fmaf(sc.a_hi, h23.x, -sc.b_hi), xh.z, ph);
      ph = __builtin_fmaf(__builtin_fmaf(sc.a_hi, h23.y, -sc.b_hi), xh.w, ph);
      __builtin_amdgcn_sched_barrier(0);
    }
    acc += active ? pl + ph : 0.0f;
    if (st != ns - 1) return;
    const float v = wave_sum(acc);
    if (lane == 0) p.y[l][row] = v;
    acc = 0.0f;
  };

  // x staging: thread t holds x[16t .. 16t + 15] of one layer (k <= 16 NT).
  const bool stager = 16 * t < k;
  f4_t xv[4];
  auto load_x = [&](int l) {
    if (stager) {
      const f4_t* src = reinterpret_cast<const f4_t*>(p.x[l] + 16 * t);
      xv[0] = src[0];
      xv[1] = src[1];
      xv[2] = src[2];
      xv[3] = src[3];
    }
  };
  auto store_x = [&](int l) {
    if (stager) {
      f4_t* dst = reinterpret_cast<f4_t*>(smem + (l & 1) * xst + xs_index(16 * t));
      dst[0] = xv[0];
      dst[1] = xv[1];
      dst[2] = xv[2];
      dst[3] = xv[3];
    }
  };

  // The next item (possibly the next layer's first) is issued before each
  // compute; the two register sets alternate by item parity, each named
  // statically in its own branch, so no set is copied while its loads are in
  // flight.  (A third set, two items ahead, measured slower: 30.4 against
  // 29.0 us for eight 4096 x 4096 layers; the kernel is bound by its VALU
  // and LDS work per weight, not by load latency.)
  WRegs<1, 1, 4> bufA, bufB;
  load_x(0);
  if (jobs > 0) issue(0, bufA);
  store_x(0);
  __syncthreads();
  int j = 0;
  for (int l = 0; l < layers; ++l) {
    if (l + 1 < layers) load_x(l + 1);
    for (int e = 0; e < per_layer; ++e, ++j) {
      if (j & 1) {
        if (j + 1 < jobs) issue(j + 1, bufA);
        compute(j, bufB);
      } else {
        if (j + 1 < jobs) issue(j + 1, bufB);
        compute(j, bufA);
      }
    }
    if (l + 1 < layers) {
      // Buffer (l + 1) & 1 was last read in layer l - 1, which every wave
      // finished before the previous barrier.
      store_x(l + 1);
      __syncthreads();
    }
  }
}

// Per-device launch facts, read once: CU count and LDS per CU; per kernel,
// the workgroups per CU that registers and wave slots allow (LDS above 64 KiB
// needs an opt-in per kernel and device).
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];
std::atomic<int> g_lds_per_cu[kMaxDevices];

hipError_t device_facts(int dev, int* cus, int* lds_per_cu) {
  int c = g_cu_count[dev].load(std::memory_order_acquire);
  int l = g_lds_per_cu[dev].load(std::memory_order_acquire);
  if (c == 0 || l == 0) {
    hipError_t e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&l, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
    if (e != hipSuccess) return e;
    g_cu_count[dev].store(c, std::memory_order_release);
    g_lds_per_cu[dev].store(l, std::memory_order_release);
  }
  *cus = c;
  *lds_per_cu = l;
  return hipSuccess;
}

// Workgroups of one GEMV launch (per layer for k_gemv_layers): enough for
// every row set, at most the resident workgroups of the whole chip (the waves
// are persistent).  Sets the kernel's LDS attribute on first use per device.
template <int MT, int R, bool GLU, int NWV, typename K>
hipError_t gemv_grid(K kern, std::atomic<int>* resident, int n, int k, int* grid, size_t* lds_out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  int cus = 0, lds_per_cu = 0;
  e = device_facts(dev, &cus, &lds_per_cu);
  if (e != hipSuccess) return e;
  int occ = resident[dev].load(std::memory_order_acquire);
  if (occ == 0) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(gemv_lds_bytes(MT, kXChunk<MT>)));
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, 64 * NWV, 0);
    if (e != hipSuccess) return e;
    occ = occ < 1 ? 1 : occ;
    resident[dev].store(occ, std::memory_order_release);
  }
  const size_t lds = gemv_lds_bytes(MT, min(k, kXChunk<MT>));
  const int by_lds = static_cast<int>(static_cast<size_t>(lds_per_cu) / lds);
  const int per_cu = max(1, min(occ, by_lds));
  const int nsets = (n + R - 1) / R;
  const int need = (nsets + NWV - 1) / NWV;
  // The gate/up pair keeps its dots in registers across K chunks, so above
  // one chunk every wave gets at most one row set.
  const bool one_set = GLU && k > kXChunk<MT>;
  *grid = one_set ? need : min(need, per_cu * cus);
  *lds_out = lds;
  return hipSuccess;
}

template <int MT, int R, bool GLU, int NWV, int FMT = 4>
hipError_t launch(const uint8_t* w, const uint8_t* w2, const float* x, float* y, int m, int n,
                  int k, hipStream_t stream) {
  static std::atomic<int> resident[kMaxDevices];  // workgroups per CU, LDS aside
  const auto kern = &k_gemv_q4k<MT, R, GLU, NWV, FMT>;
  int grid = 0;
  size_t lds = 0;
  const hipError_t e = gemv_grid<MT, R, GLU, NWV>(kern, resident, n, k, &grid, &lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * NWV), lds, stream, w, w2, x, y, m, n, k);
  return hipGetLastError();
}

hipError_t launch_layers(const LayerPtrs& p, int layers, int n, int k, hipStream_t stream) {
  static std::atomic<int> set[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  int cus = 0, lds_per_cu = 0;
  e = device_facts(dev, &cus, &lds_per_cu);
  if (e != hipSuccess) return e;
  const size_t lds = 2 * static_cast<size_t>(xs_stride(k)) * sizeof(float);
  if (!set[dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemv_layers),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(kLayersLdsBytes));
    if (e != hipSuccess) return e;
    set[dev].store(1, std::memory_order_release);
  }
  // One workgroup per CU at most (persistent), fewer when the layers have
  // fewer rows than the chip has waves.
  const int need = (n + kLayerWaves - 1) / kLayerWaves;
  const int grid = max(1, min(need, cus));
  hipLaunchKernelGGL(k_gemv_layers, dim3(grid), dim3(64 * kLayerWaves), lds, stream, p, layers,
                     n, k);
  return hipGetLastError();
}

// The decode kernel for k <= 16384: one to four K steps.
template <int NW, bool GLU, int FMT>
hipError_t launch_decode(const uint8_t* w, const uint8_t* w2, const float* x, float* y, int n,
                         int k, hipStream_t stream) {
  constexpr int RW = GLU ? NW / 2 : NW;
  const dim3 grid((n + RW - 1) / RW), block(64 * NW);
  if (k <= 4096)
    hipLaunchKernelGGL((k_gemv_decode<NW, 1, GLU, FMT>), grid, block, 0, stream, w, w2, x, y, n, k);
  else if (k <= 2 * 4096)
    hipLaunchKernelGGL((k_gemv_decode<NW, 2, GLU, FMT>), grid, block, 0, stream, w, w2, x, y, n, k);
  else if (k <= 3 * 4096)
    hipLaunchKernelGGL((k_gemv_decode<NW, 3, GLU, FMT>), grid, block, 0, stream, w, w2, x, y, n, k);
  else
    hipLaunchKernelGGL((k_gemv_decode<NW, 4, GLU, FMT>), grid, block, 0, stream, w, w2, x, y, n, k);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_gemv_passes(const uint8_t* w, const float* x, float* y, int64_t m, int64_t n,
                              int64_t k, hipStream_t stream) {
  // Batches below kGemvSplitMinM rows: one pass over W.
  const int mm = static_cast<int>(m);
  const int ni = static_cast<int>(n), ki = static_cast<int>(k);
  if (mm == 1) {
    // One row per wave.  k <= 16384 takes the decode kernel (one x staging
    // per workgroup of kDecodeWaves rows; Q4_K 14336 x 4096: 9.6 us against
    // 11.3-11.9 for the general kernel below).  Past that, matrices of up to
    // kGemvWideRows rows take the general kernel at 16 waves per workgroup;
    // taller ones 8 waves.
    if (ki <= 4 * 4096) return launch_decode<kDecodeWaves, false, FMT>(w, w, x, y, ni, ki, stream);
    if (n <= kGemvWideRows)
      return launch<1, kGemvRowsPerWave, false, 16, FMT>(w, w, x, y, mm, ni, ki, stream);
    return launch<1, kGemvRowsPerWave, false, 8, FMT>(w, w, x, y, mm, ni, ki, stream);
  }
  if (mm == 2) return launch<2, 2, false, 4, FMT>(w, w, x, y, mm, ni, ki, stream);
  return launch<4, 2, false, 4, FMT>(w, w, x, y, mm, ni, ki, stream);
}

}  // namespace

// Batches from kGemvSplitMinM rows take the split-bf16 MFMA kernel
// (k_gemv_split.hip); smaller ones the fp32 FMA passes.
hipError_t launch_gemv(const uint8_t* w, const float* x, float* y, int64_t m, int64_t n,
                       int64_t k, hipStream_t stream) {
  if (gemv_split_supported(m)) return launch_gemv_split(w, x, y, m, n, k, stream);
  return launch_gemv_passes<4>(w, x, y, m, n, k, stream);
}

hipError_t launch_q5k_gemv(const uint8_t* w, const float* x, float* y, int64_t m, int64_t n,
                           int64_t k, hipStream_t stream) {
  if (gemv_split_supported(m)) return launch_q5k_gemv_split(w, x, y, m, n, k, stream);
  return launch_gemv_passes<5>(w, x, y, m, n, k, stream);
}

hipError_t launch_gemv_layers(const uint8_t* const* w, const float* const* x, float* const* y,
                              int64_t layers, int64_t n, int64_t k, hipStream_t stream) {
  LayerPtrs p = {};
  for (int64_t l = 0; l < layers; ++l) {
    p.w[l] = w[l];
    p.x[l] = x[l];
    p.y[l] = y[l];
  }
  return launch_layers(p, static_cast<int>(layers), static_cast<int>(n), static_cast<int>(k),
                       stream);
}

hipError_t launch_gateup_swiglu(const uint8_t* w_gate, const uint8_t* w_up, const float* x,
                                float* h, int64_t d_model, int64_t d_ff, hipStream_t stream) {
  if (d_model <= 4 * 4096)
    return launch_decode<kDecodeGluWaves, true, 4>(w_gate, w_up, x, h, static_cast<int>(d_ff),
                                                static_cast<int>(d_model), stream);
  return launch<1, kGateUpRowsPerWave, true, 8>(w_gate, w_up, x, h, 1, static_cast<int>(d_ff),
                                                static_cast<int>(d_model), stream);
}

}  // namespace q4k
