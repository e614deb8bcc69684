// k_gemm.hip -- prefill GEMM Y = X W^T on Q4_K weights with bf16 MFMA.
//
// The tile GEMM of the prefill shape ("Writing an ESIMD Fused Kernel From
// Reverse-Engineered Assembly", "SLM-Tiled GEMM and Graph Recording": a
// shared-memory tiled GEMM; the PR page "CPU kernel parity ..." pairs each
// decode kernel with a tile kernel for prompt processing).  The Q4_K scale
// changes every 32 weights along K, so it cannot be folded into an output
// epilogue: each weight tile is dequantized before the contraction.
//
// Design for gfx950:
//   * workgroup = 4 waves, tile BM x BN with BN = 128 weight rows; waves are
//     arranged WAVES_M x WAVES_N, each owning (32*TI) x (32*TJ) outputs as
//     TI x TJ accumulators of v_mfma_f32_32x32x16_bf16.
//   * K advances 64 weights per step = one quant group of one super-block
//     (32 low nibbles of sub-block 2g, 32 high nibbles of 2g+1).
//   * W tile: each of the 256 threads loads the block header and 16 quant
//     bytes of one row, dequantizes 32 weights to bf16 (round to nearest
//     even of the exact fp32 weight) and writes them to LDS; the tile is
//     double-buffered, one barrier per step, and the loads run two steps
//     ahead of the MFMAs that consume them.
//   * X fragments go straight from global memory into MFMA operand layout:
//     a 16-byte load per lane per K16 slice, no LDS pass.  Within a 64-wide
//     step lane half h and slice kk hold physical k = 32h + 8kk + (0..7) for
//     both operands (the MFMA sums over k, so any common assignment is the
//     same contraction); a lane therefore reads 64 contiguous bytes of its X
//     row per step.
//   * optional split-K over blockIdx.z accumulates with fp32 atomics into a
//     zeroed Y (used when the output tile count cannot fill 256 CUs).
#include <hip/hip_runtime.h>

#include "lds_copy.h"
#include "q4k_device.h"
#include "q4k_launch.h"

namespace q4k {
namespace {

typedef float f16x_t __attribute__((ext_vector_type(16)));

constexpr int kBN = 128;       // weight rows per tile
constexpr int kBK = 64;        // weights per K step (one quant group)
constexpr int kLdsStride = 72; // bf16 per LDS row: 64 + 8 pad (144 B rows)

template <int WAVES_M, int WAVES_N, int TI, int TJ, int MINB, int FMT = 4>
__global__ __launch_bounds__(256, MINB) void k_gemm_q4k(const uint8_t* __restrict__ w,
                                                        const uint16_t* __restrict__ x,
                                                        float* __restrict__ y, int m, int n, int k,
                                                        int steps_per_split, int atomic_out) {
  static_assert(WAVES_M * WAVES_N == 4, "four waves per workgroup");
  static_assert(WAVES_N * 32 * TJ == kBN, "the tile fill covers 128 weight rows");
  constexpr int BM = WAVES_M * 32 * TI;
  __shared__ __attribute__((aligned(16))) uint16_t ws[2][kBN * kLdsStride];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;
  const int half = lane >> 5;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * kBN;
  const int kb_count = k >> 8;
  const int steps = k / kBK;
  const int s_begin = blockIdx.z * steps_per_split;
  const int s_end = min(steps, s_begin + steps_per_split);
  if (s_begin >= s_end) return;  // uniform over the workgroup, before any barrier

  // Tile-fill role: weight row f_row of the tile, 16-byte half f_hh of the group.
  const int f_row = t >> 1;
  const int f_hh = t & 1;
  constexpr int kBB = block_bytes<FMT>();
  const uint8_t* f_base = w + static_cast<size_t>(min(n0 + f_row, n - 1)) * kb_count * kBB;

  // A-operand role: rows of X this lane feeds (clamped; clamped rows are not stored).
  const uint16_t* a_ptr[TI];
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const int row = min(m0 + wm * 32 * TI + 32 * i + (lane & 31), m - 1);
    a_ptr[i] = x + static_cast<size_t>(row) * k + 32 * half;
  }

  f16x_t acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Loads past the last step re-read the last step (results unused) so the
  // pipeline needs no branches.
  // Q5_K also loads the 16 high-bit bytes of this thread's 32 weights (qh is
  // unused for Q4_K).
  auto load_w = [&](int s, uint4& hd, uint4& q, uint4& qh) {
    const int sc = min(s, s_end - 1);
    const uint8_t* p = f_base + static_cast<size_t>(sc >> 2) * kBB;
    hd = load16(p);
    if constexpr (FMT == 5) {
      q = load16(p + kQ5QuantOffset + 32 * (sc & 3) + 16 * f_hh);
      qh = load16(p + kQ5HighOffset + 16 * f_hh);
    } else {
      q = load16(p + 16 + 32 * (sc & 3) + 16 * f_hh);
      qh = q;
    }
  };
  auto load_x = [&](int s, uint4 (&xr)[TI][4]) {
    const int sc = min(s, s_end - 1);
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const uint16_t* p = a_ptr[i] + static_cast<size_t>(sc) * kBK;
#pragma unroll
      for (int c = 0; c < 4; ++c) xr[i][c] = *reinterpret_cast<const uint4*>(p + 8 * c);
    }
  };
  auto store_w = [&](int buf, int s, const uint4& hd, const uint4& q, const uint4& qh) {
    GroupScales sc = group_scales(hd, s & 3);
    uint32_t lo8[8], hi8[8];
    if constexpr (FMT == 5) {
      sc.a_lo *= 1.0f / kNibbleUnscale;  // exact integers, not q * 2^-9
      sc.a_hi *= 1.0f / kNibbleUnscale;
      dequant16_bf16_q5(q, qh, sc, s & 3, lo8, hi8);
    } else {
      dequant16_bf16(q, sc, lo8, hi8);
    }
    uint16_t* dst = &ws[buf][f_row * kLdsStride + 16 * f_hh];
    *reinterpret_cast<uint4*>(dst) = make_uint4(lo8[0], lo8[1], lo8[2], lo8[3]);
    *reinterpret_cast<uint4*>(dst + 8) = make_uint4(lo8[4], lo8[5], lo8[6], lo8[7]);
    *reinterpret_cast<uint4*>(dst + 32) = make_uint4(hi8[0], hi8[1], hi8[2], hi8[3]);
    *reinterpret_cast<uint4*>(dst + 40) = make_uint4(hi8[4], hi8[5], hi8[6], hi8[7]);
  };
  auto mfma_step = [&](int buf, const uint4 (&xr)[TI][4]) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8_t bfr[TJ];
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int nrow = wn * 32 * TJ + 32 * j + (lane & 31);
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(
            &ws[buf][nrow * kLdsStride + 32 * half + 8 * kk]);
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

  // Software pipeline, unrolled by two so that no register that a load is
  // still writing is ever copied (a copy would force a wait on the load):
  // at step s the MFMAs read LDS buffer s%2 and X registers set s%2, while
  // the weights of step s+1 are dequantized into the other LDS buffer and the
  // X fragments of step s+2 and raw weights of step s+2 are fetched.
  uint4 xA[TI][4], xB[TI][4], hA, qA, eA, hB, qB, eB;  // e: Q5_K high bits
  load_w(s_begin, hA, qA, eA);
  load_x(s_begin, xA);
  load_x(s_begin + 1, xB);
  store_w(0, s_begin, hA, qA, eA);
  load_w(s_begin + 1, hB, qB, eB);
  load_w(s_begin + 2, hA, qA, eA);
  __syncthreads();
  for (int s = s_begin; s < s_end; s += 2) {
    mfma_step(0, xA);
    load_x(s + 2, xA);
    if (s + 1 < s_end) store_w(1, s + 1, hB, qB, eB);
    load_w(s + 3, hB, qB, eB);
    __syncthreads();
    if (s + 1 >= s_end) break;
    mfma_step(1, xB);
    load_x(s + 3, xB);
    if (s + 2 < s_end) store_w(0, s + 2, hA, qA, eA);
    load_w(s + 4, hA, qA, eA);
    __syncthreads();
  }

  // Accumulator r of a 32x32 tile holds row 8*(r/4) + 4*half + r%4, column lane%32.
#pragma unroll
  for (int i = 0; i < TI; ++i) {
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int col = n0 + wn * 32 * TJ + 32 * j + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 32 * TI + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
        if (row < m && col < n) {
          float* dst = y + static_cast<size_t>(row) * n + col;
          if (atomic_out) {
            unsafeAtomicAdd(dst, acc[i][j][r]);
          } else {
            *dst = acc[i][j][r];
          }
        }
      }
    }
  }
}

// Zero fill for split-K outputs (a kernel, not a memset node, so that a
// captured graph replays it faithfully).
__global__ __launch_bounds__(256) void k_zero_f32(float* __restrict__ y, size_t count) {
  const size_t i = (static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i + 4 <= count) {
    *reinterpret_cast<f4_t*>(y + i) = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
  } else {
    for (size_t j = i; j < count; ++j) y[j] = 0.0f;
  }
}

template <int WAVES_M, int WAVES_N, int TI, int TJ, int MINB, int FMT = 4>
hipError_t launch(const uint8_t* w, const uint16_t* x, float* y, int m, int n, int k,
                  int splits_wanted, hipStream_t stream) {
  constexpr int BM = WAVES_M * 32 * TI;
  const int tiles_m = (m + BM - 1) / BM;
  const int tiles_n = (n + kBN - 1) / kBN;
  const int steps = k / kBK;
  int splits = splits_wanted < 1 ? 1 : splits_wanted;
  if (splits > steps) splits = steps;
  const int per = (steps + splits - 1) / splits;
  splits = (steps + per - 1) / per;
  if (splits > 1) {
    const size_t count = static_cast<size_t>(m) * n;
    const size_t grid = (count / 4 + 256) / 256;
    hipLaunchKernelGGL(k_zero_f32, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, y,
                       count);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k_gemm_q4k<WAVES_M, WAVES_N, TI, TJ, MINB, FMT>), dim3(tiles_n, tiles_m, splits),
                     dim3(256), 0, stream, w, x, y, m, n, k, per, splits > 1 ? 1 : 0);
  return hipGetLastError();
}


// ------------------------------------------------------------ large tiles
// 128 x 256 output tiles for prefill GEMMs with many tiles (m=512, n=14336:
// 224 tiles).  The weights never pass through LDS as bf16: each wave
// dequantizes its MFMA B fragments straight into registers.
//   * 4 waves = 2 (K parity) x 2 (N halves).  Every wave owns all 128 rows x
//     128 columns (4 x 4 accumulators of v_mfma_f32_32x32x16_bf16, 256
//     AGPRs) and, in each 64-wide K step (one quant group g), only the
//     sub-block of its parity: low nibbles (sub-block 2g) or high nibbles
//     (2g+1).  Every weight is dequantized once per workgroup; the two K
//     halves are summed through LDS at the end.
//   * within a step, lane half h of a wave holds the 16 quant bytes
//     16h .. 16h+15 of its column; MFMA slice u (0, 1) uses bytes 8u .. 8u+7
//     of that half, so slice u, lane half h covers k = 32 p + 16 h + 8 u + (0..7)
//     for parity p.  The X fragment of the same lanes reads those k.
//   * global -> LDS traffic is direct (global_load_lds_dwordx4), issued from
//     inline assembly with explicit waits: X (128 rows x 64 k = 16 KiB per
//     step) through a 5-slot ring, 5 steps ahead; whole 144-byte super-blocks
//     of the 256 weight rows (36 KiB) through a 2-slot ring, issued at the
//     last step of the super-block before the one that needs them.
//   * LDS X rows are 128 bytes with XOR-swizzled 16-byte chunks (conflict-
//     free fragment reads); weight rows keep their 144-byte record, whose
//     36-dword stride spreads 16 consecutive rows over all 64 banks.
//   * K starts at a super-block that depends on the N-tile only: the M-tiles
//     that share a weight tile walk K in step, and the N-tiles that share X
//     rows start at different offsets.  When the tile grid allows, all
//     M-tiles of an N-tile run on one XCD, so its L2 serves their weight reads.
constexpr int kWBM = 128, kWBN = 256;
constexpr int kWXSlot = kWBM * 128;          // bytes per X slot (one step)
constexpr int kWWSlot = kWBN * kBlockBytes;  // bytes per weight slot (one super-block)
constexpr int kWXSlots = 5;
constexpr int kWWOff = kWXSlots * kWXSlot;
constexpr int kWLds = kWXSlots * kWXSlot + 2 * kWWSlot;  // 155648 bytes
static_assert(kWLds <= 160 * 1024, "LDS budget of one workgroup");
static_assert(2 * 2 * 32768 <= kWLds, "the K-half exchange reuses the rings");

struct XFrag {
  bf16x8_t a[2][4];  // [slice u][M block i]
};

__global__ __launch_bounds__(256, 1) void k_gemm_q4k_128x256(const uint8_t* __restrict__ w,
                                                             const uint16_t* __restrict__ x,
                                                             float* __restrict__ y, int m, int n,
                                                             int k, int tiles_m, int tiles_n,
                                                             int xcd_gm) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kWLds];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int h = lane >> 5;
  const int c32 = lane & 31;
  const int kp = wave >> 1;  // K parity: 0 = low nibbles, 1 = high nibbles
  const int wn = wave & 1;   // N half
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, xcd_gm, tm, tn);
  const int m0 = tm * kWBM, n0 = tn * kWBN;
  const int nsb = k >> 8;                     // super-blocks along K
  const int nst = k >> 6;                     // 64-wide steps
  const uint32_t row_bytes = static_cast<uint32_t>(nsb) * kBlockBytes;
  // The tile's first weight row, in 64 bits; offsets inside the tile's 256
  // rows stay below 2^32 (k <= 2^24, checked by the C ABI).
  const uint8_t* const wt = w + static_cast<size_t>(n0) * row_bytes;
  // Super-block of step group S (indices past the end repeat the last).  Every
  // tile walks K from super-block 0, so the tiles of one XCD that share X rows
  // read the same K window of X at the same time and find it in their L2.
  auto phys_sb = [&](int S) { return min(S, nsb - 1); };

  // X copy q of this wave fills tile rows 8 (4 wave + q) .. +7; lane ->
  // (row, LDS chunk lane % 8) holding X chunk (lane % 8) ^ swz(row).
  const uint16_t* xsrc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 8 * (wave * 4 + q) + (lane >> 3);
    const int c = (lane & 7) ^ swz(row);
    xsrc[q] = x + static_cast<size_t>(min(m0 + row, m - 1)) * k + 8 * c;
  }
  // Weight copy i of this wave fills 16-byte unit P = 64 (9 wave + i) + lane
  // of the slot: row P / 9, part P % 9 of its 144-byte super-block.
  uint32_t woff[9];
#pragma unroll
  for (int i = 0; i < 9; ++i) {
    const int P = (wave * 9 + i) * 64 + lane;
    const int col = (P * 7282) >> 16;  // P / 9 for P < 2304
    woff[i] = static_cast<uint32_t>(min(col, n - 1 - n0)) * row_bytes + (P - col * 9) * 16;
  }
  const uint32_t lds0 = lds_address(smem);
  auto copy_x = [&](int s, int slot) {
    const int sc = min(s, nst - 1);
    const int ps = 4 * phys_sb(sc >> 2) + (sc & 3);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      copy16_to_lds(xsrc[q] + static_cast<size_t>(ps) * 64,
                    __builtin_amdgcn_readfirstlane(lds0 + slot * kWXSlot + (wave * 4 + q) * 1024));
  };
  auto copy_w = [&](int S, int slot) {
    const uint8_t* base = wt + static_cast<size_t>(phys_sb(S)) * kBlockBytes;
#pragma unroll
    for (int i = 0; i < 9; ++i)
      copy16_to_lds(base + woff[i], __builtin_amdgcn_readfirstlane(
                                        lds0 + kWWOff + slot * kWWSlot + (wave * 9 + i) * 1024));
  };
  // Fragments: X slices of the wave's parity; quant half h and header of its columns.
  auto read_x = [&](int slot, XFrag& A) {
    const uint8_t* xb = smem + slot * kWXSlot;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 32 * i + c32;
        const int ch = kp * 4 + 2 * h + u;
        A.a[u][i] = *reinterpret_cast<const bf16x8_t*>(xb + r * 128 + ((ch ^ swz(r)) << 4));
      }
  };
  auto read_q = [&](int slot, int g, uint4 (&Q)[4]) {
    const uint8_t* wb = smem + kWWOff + slot * kWWSlot;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = wn * 128 + 32 * j + c32;
      Q[j] = *reinterpret_cast<const uint4*>(wb + col * kBlockBytes + 16 + 32 * g + 16 * h);
    }
  };
  auto read_hdr = [&](int slot, uint4 (&H)[4]) {
    const uint8_t* wb = smem + kWWOff + slot * kWWSlot;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = wn * 128 + 32 * j + c32;
      H[j] = *reinterpret_cast<const uint4*>(wb + col * kBlockBytes);
    }
  };
  // sa[g][j], sb[g][j]: a = d*sc*2^9 and b = dmin*mn of sub-block 2g + kp of column block j.
  auto scales = [&](const uint4 (&H)[4], float (&sa)[4][4], float (&sb)[4][4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 hd = H[j];
      const uint32_t sc_lo = hd.y & 0x3F3F3F3Fu;
      const uint32_t mn_lo = hd.z & 0x3F3F3F3Fu;
      const uint32_t sc_hi = (hd.w & 0x0F0F0F0Fu) | ((hd.y >> 2) & 0x30303030u);
      const uint32_t mn_hi = ((hd.w >> 4) & 0x0F0F0F0Fu) | ((hd.z >> 2) & 0x30303030u);
      const float d = half_bits_to_float(hd.x & 0xFFFFu) * kNibbleUnscale;
      const float dmin = half_bits_to_float(hd.x >> 16);
      const int sh = 8 * kp;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t scw = (g < 2 ? sc_lo : sc_hi) >> (sh + 16 * (g & 1));
        const uint32_t mnw = (g < 2 ? mn_lo : mn_hi) >> (sh + 16 * (g & 1));
        sa[g][j] = d * static_cast<float>(scw & 0xFFu);
        sb[g][j] = dmin * static_cast<float>(mnw & 0xFFu);
      }
    }
  };
  const int nshift = 4 * kp;
  auto dequant = [&](const uint4 (&Q)[4], int u, const float (&a)[4], const float (&b)[4],
                     bf16x8_t (&B)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      B[j] = dequant8_bf16(u ? Q[j].z : Q[j].x, u ? Q[j].w : Q[j].y, nshift, a[j], b[j]);
  };
  f16x_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  auto mfmas = [&](const XFrag& A, int u, const bf16x8_t (&B)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A.a[u][i], B[j], acc[i][j], 0, 0, 0);
  };

  // Copies per wave: X 4 per step, weights 9 per super-block.  Prologue:
  // W(0), X(0..4), W(1); W(0) and X(0) land, then X(1).
  copy_w(0, 0);
#pragma unroll
  for (int s = 0; s < kWXSlots; ++s) copy_x(s, s);
  copy_w(1, 1);
  wait_copies_barrier<4 * 4 + 9>();
  XFrag A0, A1;
  uint4 Q0[4], Q1[4], H[4];
  float sa[4][4], sb[4][4];
  read_hdr(0, H);
  read_q(0, 0, Q0);
  read_x(0, A0);
  wait_copies_barrier<3 * 4 + 9>();
  scales(H, sa, sb);
  bf16x8_t B0[4];
  dequant(Q0, 0, sa[0], sb[0], B0);

  int xs = 0;  // X slot of step s
  int ws = 0;  // weight slot of super-block S
  // Step s (phase p = s % 4 of super-block S): issue X(s+5) and, at phase 3,
  // W(S+2); read the fragments of step s+1; MFMAs of step s, the weights of
  // slice 1 and of step s+1's slice 0 dequantized in between.  At the end of
  // the step every copy issued up to step s-3 has landed (X(s+2), and from
  // phase 2 on W(S+1)).
  auto step = [&](int s, int p, XFrag& Ac, uint4 (&Qc)[4], XFrag& An, uint4 (&Qn)[4]) {
    const int xn = xs == kWXSlots - 1 ? 0 : xs + 1;
    const int ws1 = ws ^ 1;
    copy_x(s + kWXSlots, xs);
    if (p == 3) copy_w((s >> 2) + 2, ws);
    read_x(xn, An);
    if (p < 3) {
      read_q(ws, p + 1, Qn);
    } else {
      read_q(ws1, 0, Qn);
      read_hdr(ws1, H);
    }
    __builtin_amdgcn_sched_barrier(0);
    bf16x8_t B1[4];
    dequant(Qc, 1, sa[p], sb[p], B1);
    mfmas(Ac, 0, B0);
    if (p < 3) {
      dequant(Qn, 0, sa[p + 1], sb[p + 1], B0);
    } else {
      scales(H, sa, sb);
      dequant(Qn, 0, sa[0], sb[0], B0);
    }
    mfmas(Ac, 1, B1);
    // One MFMA, then five VALU instructions, so the dequantization runs
    // under the matrix core.
#pragma unroll
    for (int q = 0; q < 32; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (p == 2)
      wait_copies_barrier<3 * 4>();
    else
      wait_copies_barrier<3 * 4 + 9>();
    __builtin_amdgcn_sched_barrier(0);
    xs = xn;
    if (p == 3) ws = ws1;
  };
  for (int s = 0; s < nst; s += 4) {
    step(s, 0, A0, Q0, A1, Q1);
    step(s + 1, 1, A1, Q1, A0, Q0);
    step(s + 2, 2, A0, Q0, A1, Q1);
    step(s + 3, 3, A1, Q1, A0, Q0);
  }
  // No copy into this workgroup's LDS may outlive it; the rings are reused below.
  wait_copies_barrier<0>();

  // Sum the K halves: parity 1 hands rows 0..63 to parity 0, parity 0 hands
  // rows 64..127 to parity 1; each lane moves its own accumulator registers.
  uint8_t* const ex_out = smem + (kp == 1 ? 0 : 65536) + wn * 32768;
  const uint8_t* const ex_in = smem + (kp == 0 ? 0 : 65536) + wn * 32768;
  auto put = [&](int il, const f16x_t (&row)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<f4_t*>(ex_out + ((il * 4 + j) * 4 + r4) * 1024 + lane * 16) =
            f4_t{row[j][4 * r4], row[j][4 * r4 + 1], row[j][4 * r4 + 2], row[j][4 * r4 + 3]};
  };
  if (kp == 1) {
    put(0, acc[0]);
    put(1, acc[1]);
  } else {
    put(0, acc[2]);
    put(1, acc[3]);
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // Accumulator r of a 32x32 tile holds row 8*(r/4) + 4*h + r%4, column lane%32.
  auto finish = [&](int il, int i, const f16x_t (&row)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 128 + 32 * j + c32;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f4_t o = *reinterpret_cast<const f4_t*>(ex_in + ((il * 4 + j) * 4 + r4) * 1024 + lane * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * r4 + e;
          const int row_g = m0 + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
          if (row_g < m && col < n) y[static_cast<size_t>(row_g) * n + col] = row[j][r] + o[e];
        }
      }
    }
  };
  if (kp == 0) {
    finish(0, 0, acc[0]);
    finish(1, 1, acc[1]);
  } else {
    finish(0, 2, acc[2]);
    finish(1, 3, acc[3]);
  }
}

// ------------------------------------------------------------ K-slice tiles
// (32 TI) x (32 NJ TI) output tiles with K split four ways inside the
// workgroup, for grids that the 128 x 256 tiles cannot fill without splitting
// K across workgroups (m=512, n=4096: TI=NJ=2, 256 tiles of 64 x 128; m=256,
// n=4096: TI=2, NJ=1, 256 tiles of 64 x 64; batches of at most 32 rows take
// the streaming kernel of k_gemm_stream.hip).  Splitting K across workgroups
// would need fp32 atomics (about one per L2 channel per clock: 29 us measured
// for the 8 M adds of the m=512, n=4096 output split four ways) or a second
// pass.
//   * 4 TI waves = 4 K slices x TI N halves.  Wave (kq, wn) owns all 32 TI
//     rows x 32 NJ columns of its half (TI x NJ accumulators) and, in every 64-wide
//     K step, k = 32 p + 16 b + 8 h + (0..7) with p = kq / 2 (nibble parity),
//     b = kq % 2 (byte half) and h the lane half: the low or high nibbles of
//     quant bytes 16 b + 8 h .. +7.  Every weight is dequantized once per
//     workgroup; the four K slices are summed through LDS at the end.
//   * copies as in the 128 x 256 kernel: X (32 TI rows x 64 k) through a
//     9-slot ring, whole super-block records of the weight rows (144 bytes for
//     Q4_K, 176 for Q5_K) through a 4- or 3-slot ring issued three super-blocks
//     ahead; per wave one X copy per step and three weight copies per
//     super-block.  Q5_K lanes also read the 8 high-bit bytes that match their
//     quant bytes and widen 5-bit bytes exactly (v_cvt_f32_ubyte).
//   * the sub-block scales of a super-block are decoded once per workgroup
//     (thread t: row t / 4, group t % 4) into LDS; waves read the (a, b) pairs
//     of their parity.
//   * quant bytes are read two steps ahead of their dequantization, which runs
//     under the MFMAs of the step before their use.
template <int TI, int NJ, int FMT = 4>
struct KSlice {
  static constexpr int BM = 32 * TI, BN = 32 * NJ * TI, Threads = 256 * TI;
  static constexpr int BB = block_bytes<FMT>();  // 144 (Q4_K) or 176 (Q5_K)
  static constexpr int Units = BB / 16;          // 16-byte copy units per record
  static constexpr int WaveUnits = 8 * NJ * Units;  // weight units copied per wave
  static constexpr int WCopies = (WaveUnits + 63) / 64;  // copies per wave per super-block
  static constexpr int XSlot = BM * 128;
  static constexpr int WSlot = BN * BB;
  static constexpr int XSlots = 9;
  // Slot S % WSlots holds super-block S.  Its last reads are at phase 1 of S and
  // super-block S + 3 is copied at phase 3, so three slots suffice; Q4_K keeps
  // a fourth (the LDS has room for it).
  static constexpr int WSlots = FMT == 5 ? 3 : 4;
  static constexpr int WOff = XSlots * XSlot;
  static constexpr int SOff = WOff + WSlots * WSlot;
  static constexpr int SSlot = 4 * BN * 16;  // [parity][group pair][row] x (a, b, a', b')
  static constexpr int Lds = SOff + 2 * SSlot;
  static constexpr int ExWave = TI * NJ * 4 * 1024;  // one wave's partial tile
  static_assert(Lds <= 160 * 1024, "LDS budget of one workgroup");
  static_assert(4 * TI * ExWave <= SOff, "the K-slice exchange reuses the rings");
};

template <int TI>
struct XFragT {
  bf16x8_t a[TI];  // [M block]
};

// A lane's quant bytes for one step: 8 quant bytes, and for Q5_K the 8
// matching high-bit-plane bytes (unused for Q4_K).
struct QBytes {
  uint2 q, hb;
};

template <int TI, int NJ, int FMT = 4>
__global__ __launch_bounds__(256 * TI, 1) void k_gemm_q4k_kslice(const uint8_t* __restrict__ w,
                                                                 const uint16_t* __restrict__ x,
                                                                 float* __restrict__ y, int m,
                                                                 int n, int k, int tiles_m,
                                                                 int tiles_n, int xcd_gm) {
  using C = KSlice<TI, NJ, FMT>;
  constexpr int kColsPerWave = 32 * NJ;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::Lds];
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int h = lane >> 5;
  const int c32 = lane & 31;
  const int kq = wave & 3;
  const int par = kq >> 1;   // nibble parity of this K slice
  const int bh = kq & 1;     // byte half of this K slice
  const int wn = wave >> 2;  // N half
  int tm, tn;
  tile_coords(blockIdx.x, tiles_m, tiles_n, xcd_gm, tm, tn);
  const int m0 = tm * C::BM, n0 = tn * C::BN;
  const int nsb = k >> 8, nst = k >> 6;
  const uint32_t row_bytes = static_cast<uint32_t>(nsb) * C::BB;
  // The tile's first weight row, in 64 bits; offsets inside the tile stay
  // below 2^32 (k <= 2^24, checked by the C ABI).
  const uint8_t* const wt = w + static_cast<size_t>(n0) * row_bytes;
  auto phys_sb = [&](int S) { return min(S, nsb - 1); };  // K from super-block 0 (as above)
  // X copy of this wave: tile rows 8 wave .. +7.
  const uint16_t* xsrc;
  {
    const int row = 8 * wave + (lane >> 3);
    const int c = (lane & 7) ^ swz(row);
    xsrc = x + static_cast<size_t>(min(m0 + row, m - 1)) * k + 8 * c;
  }
  // Weight copies of this wave: 16-byte units WaveUnits wave + min(64 i,
  // WaveUnits - 64) + lane of the slot (Q4_K, NJ = 2: 144 units from
  // {0, 64, 80}; Q5_K: 176 from {0, 64, 112}); the last copy repeats some
  // units of the one before, with the same data and place.
  auto unit0 = [](int i) { return min(64 * i, C::WaveUnits - 64); };
  uint32_t woff[C::WCopies];
#pragma unroll
  for (int i = 0; i < C::WCopies; ++i) {
    const int U = C::WaveUnits * wave + unit0(i) + lane;
    const int col = FMT == 5 ? U / C::Units : (U * 7282) >> 16;  // U / 9 for U < 2304
    woff[i] = static_cast<uint32_t>(min(col, n - 1 - n0)) * row_bytes + (U - col * C::Units) * 16;
  }
  const uint32_t lds0 = lds_address(smem);
  auto copy_x = [&](int s, int slot) {
    const int sc = min(s, nst - 1);
    const int ps = 4 * phys_sb(sc >> 2) + (sc & 3);
    copy16_to_lds(xsrc + static_cast<size_t>(ps) * 64,
                  __builtin_amdgcn_readfirstlane(lds0 + slot * C::XSlot + wave * 1024));
  };
  auto copy_w = [&](int S, int slot) {
    const uint8_t* base = wt + static_cast<size_t>(phys_sb(S)) * C::BB;
#pragma unroll
    for (int i = 0; i < C::WCopies; ++i)
      copy16_to_lds(base + woff[i],
                    __builtin_amdgcn_readfirstlane(lds0 + C::WOff + slot * C::WSlot +
                                                   (C::WaveUnits * wave + unit0(i)) * 16));
  };
  auto read_x = [&](int slot, XFragT<TI>& A) {
    const uint8_t* xb = smem + slot * C::XSlot;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int r = 32 * i + c32;
      const int ch = 4 * par + 2 * bh + h;
      A.a[i] = *reinterpret_cast<const bf16x8_t*>(xb + r * 128 + ((ch ^ swz(r)) << 4));
    }
  };
  // Quant bytes r = 16 bh + 8 h + (0..7) of group g, and for Q5_K the same
  // bytes of the high-bit plane (bit 2 g + parity is the fifth bit).
  auto read_q = [&](int slot, int g, QBytes (&Q)[NJ]) {
    const uint8_t* wb = smem + C::WOff + slot * C::WSlot;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int col = kColsPerWave * wn + 32 * j + c32;
      const uint8_t* rec = wb + col * C::BB;
      // 8 bytes per lane: the two lane halves read different addresses (a
      // 16-byte read that both halves share costs LDS bank conflicts).
      Q[j].q = *reinterpret_cast<const uint2*>(
          rec + (FMT == 5 ? kQ5QuantOffset : 16) + 32 * g + 16 * bh + 8 * h);
      if constexpr (FMT == 5)
        Q[j].hb = *reinterpret_cast<const uint2*>(rec + kQ5HighOffset + 16 * bh + 8 * h);
    }
  };
  auto scales_store = [&](int wslot, int ss) {
    const int col = t >> 2, g = t & 3;
    // (With NJ = 1 half the threads have no row; with NJ = 2 the test folds away,
    // so the step stays one basic block for the scheduling hints below.)
    if (C::Threads / 4 > C::BN && col >= C::BN) return;
    const uint4 hd =
        *reinterpret_cast<const uint4*>(smem + C::WOff + wslot * C::WSlot + col * C::BB);
    GroupScales gs = group_scales(hd, g);
    if constexpr (FMT == 5) {  // 5-bit quants are widened as exact integers, not q * 2^-9
      gs.a_lo *= 1.0f / kNibbleUnscale;
      gs.a_hi *= 1.0f / kNibbleUnscale;
    }
    uint8_t* sp = smem + C::SOff + ss * C::SSlot;
    *reinterpret_cast<f2_t*>(sp + ((g >> 1) * C::BN + col) * 16 + (g & 1) * 8) = f2_t{gs.a_lo, gs.b_lo};
    *reinterpret_cast<f2_t*>(sp + ((2 + (g >> 1)) * C::BN + col) * 16 + (g & 1) * 8) = f2_t{gs.a_hi, gs.b_hi};
  };
  auto scales_load = [&](int ss, float (&sa)[4][NJ], float (&sb)[4][NJ]) {
    const uint8_t* sp = smem + C::SOff + ss * C::SSlot;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int col = kColsPerWave * wn + 32 * j + c32;
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        const f4_t v = *reinterpret_cast<const f4_t*>(sp + ((par * 2 + gp) * C::BN + col) * 16);
        sa[2 * gp][j] = v.x;
        sb[2 * gp][j] = v.y;
        sa[2 * gp + 1][j] = v.z;
        sb[2 * gp + 1][j] = v.w;
      }
    }
  };
  const int nshift = 4 * par;
  auto dequant = [&](const QBytes (&Q)[NJ], int g, const float (&a)[NJ], const float (&b)[NJ],
                     bf16x8_t (&B)[NJ]) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if constexpr (FMT == 5)
        B[j] = __builtin_bit_cast(
            bf16x8_t, dequant8_bf16_q5(q5_bytes(Q[j].q.x, Q[j].hb.x, nshift, 2 * g + par),
                                       q5_bytes(Q[j].q.y, Q[j].hb.y, nshift, 2 * g + par), a[j], b[j]));
      else
        B[j] = dequant8_bf16(Q[j].q.x, Q[j].q.y, nshift, a[j], b[j]);
    }
  };
  f16x_t acc[TI][NJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  auto mfmas = [&](const XFragT<TI>& A, const bf16x8_t (&B)[NJ]) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A.a[i], B[j], acc[i][j], 0, 0, 0);
  };

  // Copies per wave: X 1 per step, weights 3 per super-block.  Step j issues
  // X(j + 9) and, at phase 3, W(j / 4 + 3); the prologue plays steps -9 .. -1.
  copy_x(0, 0);
  copy_w(0, 0);
#pragma unroll
  for (int s = 1; s <= 4; ++s) copy_x(s, s);
  copy_w(1, 1);
#pragma unroll
  for (int s = 5; s <= 8; ++s) copy_x(s, s);
  copy_w(2, 2);
  constexpr int CW = C::WCopies;
  wait_copies_barrier<8 + 2 * CW>();  // X(0), W(0) landed
  XFragT<TI> A0, A1;
  QBytes Q0[NJ], Q1[NJ];
  float sa[4][NJ], sb[4][NJ];
  scales_store(0, 0);
  read_q(0, 0, Q0);
  read_q(0, 1, Q1);
  read_x(0, A0);
  // The end of step -1: every copy of step -8 and before has landed, X(1)
  // among them (step 0 reads it).  After X(1) came X(2..8), W(1) and W(2).
  wait_copies_barrier<7 + 2 * CW>();
  scales_load(0, sa, sb);
  bf16x8_t B0[NJ], B1[NJ];
  dequant(Q0, 0, sa[0], sb[0], B0);

  int xs = 0;  // X slot of step s
  int ws = 0;  // weight slot of super-block S
  // Step s (phase p of super-block S): copies X(s+9) and at phase 3 W(S+3);
  // reads the X fragments of step s+1, the quant bytes of step s+2 (into Qb)
  // and at phase 2 decodes the scales of S+1; MFMAs of step s with Bc while
  // Bn = B(s+1) is dequantized from Qa, read one step earlier.
  auto step = [&](int s, int p, XFragT<TI>& Ac, XFragT<TI>& An, QBytes (&Qa)[NJ], QBytes (&Qb)[NJ],
                  bf16x8_t (&Bc)[NJ], bf16x8_t (&Bn)[NJ]) {
    const int xn = xs == C::XSlots - 1 ? 0 : xs + 1;
    const int ws1 = C::WSlots == 4 ? (ws + 1) & 3 : (ws == C::WSlots - 1 ? 0 : ws + 1);
    copy_x(s + C::XSlots, xs);
    if (p == 3) copy_w((s >> 2) + 3, C::WSlots == 4 ? (ws + 3) & 3 : ws);  // slot of S + 3
    read_x(xn, An);
    read_q(p < 2 ? ws : ws1, (p + 2) & 3, Qb);
    if (p == 2) scales_store(ws1, ((s >> 2) + 1) & 1);
    __builtin_amdgcn_sched_barrier(0);
    mfmas(Ac, Bc);
    if (p < 3) {
      dequant(Qa, p + 1, sa[p + 1], sb[p + 1], Bn);
    } else {
      scales_load(((s >> 2) + 1) & 1, sa, sb);
      dequant(Qa, 0, sa[0], sb[0], Bn);
    }
#pragma unroll
    for (int q = 0; q < NJ * TI; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // End of step s: every copy issued up to step s-7 has landed (X(s+2));
    // at phase 1 up to step s-6 (W(S+1), read from phase 2 on).
    if (p == 1)
      wait_copies_barrier<6 + CW>();
    else if (p == 2)
      wait_copies_barrier<7 + CW>();
    else
      wait_copies_barrier<7 + 2 * CW>();
    __builtin_amdgcn_sched_barrier(0);
    xs = xn;
    if (p == 3) ws = ws1;
  };
  for (int s = 0; s < nst; s += 4) {
    step(s, 0, A0, A1, Q1, Q0, B0, B1);
    step(s + 1, 1, A1, A0, Q0, Q1, B1, B0);
    step(s + 2, 2, A0, A1, Q1, Q0, B0, B1);
    step(s + 3, 3, A1, A0, Q0, Q1, B1, B0);
  }
  wait_copies_barrier<0>();

  // Sum the K slices: wave w writes its partial tile (TI x NJ accumulators,
  // one 1-KiB unit per 4 registers) to region w; wave (kq, wn) then finishes
  // units kq U/4 .. (kq+1) U/4 - 1 (U = 4 TI NJ) of N half wn from the four
  // regions of that half.
  uint8_t* const reg_out = smem + wave * C::ExWave;
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        *reinterpret_cast<f4_t*>(reg_out + ((i * NJ + j) * 4 + r4) * 1024 + lane * 16) =
            f4_t{acc[i][j][4 * r4], acc[i][j][4 * r4 + 1], acc[i][j][4 * r4 + 2], acc[i][j][4 * r4 + 3]};
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  constexpr int kUnitsPerWave = TI * NJ;  // U / 4
#pragma unroll
  for (int uu = 0; uu < kUnitsPerWave; ++uu) {
    const int u = kq * kUnitsPerWave + uu;
    const int i = u / (NJ * 4), j = (u >> 2) % NJ, r4 = u & 3;
    const int col = n0 + kColsPerWave * wn + 32 * j + c32;
    f4_t v = f4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int src = 0; src < 4; ++src)
      v += *reinterpret_cast<const f4_t*>(smem + (wn * 4 + src) * C::ExWave + u * 1024 + lane * 16);
    // Accumulator r of a 32x32 tile holds row 8*(r/4) + 4*h + r%4, column lane%32.
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * r4 + e;
      const int row = m0 + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
      if (row < m && col < n) y[static_cast<size_t>(row) * n + col] = v[e];
    }
  }
}

// XCD blocking of a tiles_m x tiles_n grid of bm x bn tiles (see tile_coords):
// the gm in {1, 2, 4, 8} that divides the grid and minimizes the bytes one
// XCD's workgroups stream per K element (2 per X row, 9/16 per weight row),
// or 0 if none divides it.
int xcd_groups(int tiles_m, int tiles_n, int bm, int bn) {
  return xcd_blocking(tiles_m, tiles_n, 32L * bm, 9L * bn);
}

// Split K until the grid reaches one workgroup per CU (256 on MI355X).
int splits_for(int tiles, int steps) {
  int s = 1;
  while (tiles * s * 2 <= 256 && s * 2 <= steps / 8) s *= 2;
  return s;
}

}  // namespace

hipError_t launch_gemm(const uint8_t* w, const uint16_t* x, float* y, int64_t m, int64_t n,
                       int64_t k, hipStream_t stream) {
  const int mi = static_cast<int>(m), ni = static_cast<int>(n), ki = static_cast<int>(k);
  const int steps = ki / kBK;
  const int tiles_n = (ni + kBN - 1) / kBN;
  if (mi <= 32) {
    // 64 weight rows per workgroup, each wave streaming its own super-blocks.
    if (gemm_stream_tiles(ni) >= kGemmSmallTiles) return launch_gemm_stream(w, x, y, m, n, k, stream);
    // Small batch: one 32-row slice, the four waves split the 128 weight rows.
    return launch<1, 4, 1, 1, 2>(w, x, y, mi, ni, ki, splits_for(tiles_n, steps), stream);
  }
  const int big_m = (mi + kWBM - 1) / kWBM, big_n = (ni + kWBN - 1) / kWBN;
  if (mi >= 2 * kWBM && big_m * big_n >= kGemmBigTiles) {
    // Enough 128 x 256 tiles to fill most CUs without splitting K.
    hipLaunchKernelGGL(k_gemm_q4k_128x256, dim3(big_m * big_n), dim3(256), 0, stream, w, x, y,
                       mi, ni, ki, big_m, big_n, xcd_groups(big_m, big_n, kWBM, kWBN));
    return hipGetLastError();
  }
  using Mid = KSlice<2, 2>;
  const int mid_m = (mi + Mid::BM - 1) / Mid::BM, mid_n = (ni + Mid::BN - 1) / Mid::BN;
  if (mid_m * mid_n >= kGemmMidTiles) {
    // Enough 64 x 128 tiles to fill most CUs without splitting K.
    hipLaunchKernelGGL((k_gemm_q4k_kslice<2, 2>), dim3(mid_m * mid_n), dim3(Mid::Threads), 0,
                       stream, w, x, y, mi, ni, ki, mid_m, mid_n,
                       xcd_groups(mid_m, mid_n, Mid::BM, Mid::BN));
    return hipGetLastError();
  }
  using Quad = KSlice<2, 1>;
  const int quad_m = (mi + Quad::BM - 1) / Quad::BM, quad_n = (ni + Quad::BN - 1) / Quad::BN;
  if (quad_m * quad_n >= kGemmMidTiles) {
    // 64 x 64 tiles (256 x 4096 x 4096: 23 us against 30 with split K).
    hipLaunchKernelGGL((k_gemm_q4k_kslice<2, 1>), dim3(quad_m * quad_n), dim3(Quad::Threads), 0,
                       stream, w, x, y, mi, ni, ki, quad_m, quad_n,
                       xcd_groups(quad_m, quad_n, Quad::BM, Quad::BN));
    return hipGetLastError();
  }
  // 128 x 128 tiles, two workgroups per CU.
  const int tiles = ((mi + 127) / 128) * tiles_n;
  return launch<4, 1, 1, 4, 2>(w, x, y, mi, ni, ki, splits_for(tiles, steps), stream);
}

// Q5_K: the K-slice kernels on 176-byte records where their grids fill the
// chip (as for Q4_K), else the tile kernel that dequantizes each step's weight
// tile into LDS, split K when the tile grid is small.
hipError_t launch_q5k_gemm(const uint8_t* w, const uint16_t* x, float* y, int64_t m, int64_t n,
                           int64_t k, hipStream_t stream) {
  const int mi = static_cast<int>(m), ni = static_cast<int>(n), ki = static_cast<int>(k);
  const int steps = ki / kBK;
  const int tiles_n = (ni + kBN - 1) / kBN;
  if (mi <= 32) {
    if (gemm_stream_tiles(ni) >= kGemmSmallTiles)
      return launch_q5k_gemm_stream(w, x, y, m, n, k, stream);
    return launch<1, 4, 1, 1, 2, 5>(w, x, y, mi, ni, ki, splits_for(tiles_n, steps), stream);
  }
  // The K-slice tiles serve the grids between one and a few waves of
  // workgroups; grids that Q4_K gives to its 128 x 256 tiles run faster on the
  // LDS-dequant tiles here (512 x 14336 x 4096: 116 against 152 us).
  using Mid = KSlice<2, 2, 5>;
  const int mid_m = (mi + Mid::BM - 1) / Mid::BM, mid_n = (ni + Mid::BN - 1) / Mid::BN;
  const int big_m = (mi + kWBM - 1) / kWBM, big_n = (ni + kWBN - 1) / kWBN;
  const bool big_grid = mi >= 2 * kWBM && big_m * big_n >= kGemmBigTiles;
  if (!big_grid && mid_m * mid_n >= kGemmMidTiles) {
    hipLaunchKernelGGL((k_gemm_q4k_kslice<2, 2, 5>), dim3(mid_m * mid_n), dim3(Mid::Threads), 0,
                       stream, w, x, y, mi, ni, ki, mid_m, mid_n,
                       xcd_groups(mid_m, mid_n, Mid::BM, Mid::BN));
    return hipGetLastError();
  }
  using Quad = KSlice<2, 1, 5>;
  const int quad_m = (mi + Quad::BM - 1) / Quad::BM, quad_n = (ni + Quad::BN - 1) / Quad::BN;
  if (!big_grid && quad_m * quad_n >= kGemmMidTiles) {
    hipLaunchKernelGGL((k_gemm_q4k_kslice<2, 1, 5>), dim3(quad_m * quad_n), dim3(Quad::Threads), 0,
                       stream, w, x, y, mi, ni, ki, quad_m, quad_n,
                       xcd_groups(quad_m, quad_n, Quad::BM, Quad::BN));
    return hipGetLastError();
  }
  const int tiles = ((mi + 127) / 128) * tiles_n;
  return launch<4, 1, 1, 4, 2, 5>(w, x, y, mi, ni, ki, splits_for(tiles, steps), stream);
}

}  // namespace q4k
