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

#include "q4k_device.h"
#include "q4k_launch.h"

namespace q4k {
namespace {

typedef float f16x_t __attribute__((ext_vector_type(16)));

constexpr int kBN = 128;       // weight rows per tile
constexpr int kBK = 64;        // weights per K step (one quant group)
constexpr int kLdsStride = 72; // bf16 per LDS row: 64 + 8 pad (144 B rows)

template <int WAVES_M, int WAVES_N, int TI, int TJ, int MINB>
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
  const uint8_t* f_base =
      w + static_cast<size_t>(min(n0 + f_row, n - 1)) * kb_count * kBlockBytes;

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
  auto load_w = [&](int s, uint4& hd, uint4& q) {
    const int sc = min(s, s_end - 1);
    const uint8_t* p = f_base + static_cast<size_t>(sc >> 2) * kBlockBytes;
    hd = load16(p);
    q = load16(p + 16 + 32 * (sc & 3) + 16 * f_hh);
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
  auto store_w = [&](int buf, int s, const uint4& hd, const uint4& q) {
    const GroupScales sc = group_scales(hd, s & 3);
    uint32_t lo8[8], hi8[8];
    dequant16_bf16(q, sc, lo8, hi8);
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
  uint4 xA[TI][4], xB[TI][4], hA, qA, hB, qB;
  load_w(s_begin, hA, qA);
  load_x(s_begin, xA);
  load_x(s_begin + 1, xB);
  store_w(0, s_begin, hA, qA);
  load_w(s_begin + 1, hB, qB);
  load_w(s_begin + 2, hA, qA);
  __syncthreads();
  for (int s = s_begin; s < s_end; s += 2) {
    mfma_step(0, xA);
    load_x(s + 2, xA);
    if (s + 1 < s_end) store_w(1, s + 1, hB, qB);
    load_w(s + 3, hB, qB);
    __syncthreads();
    if (s + 1 >= s_end) break;
    mfma_step(1, xB);
    load_x(s + 3, xB);
    if (s + 2 < s_end) store_w(0, s + 2, hA, qA);
    load_w(s + 4, hA, qA);
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

template <int WAVES_M, int WAVES_N, int TI, int TJ, int MINB>
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
  hipLaunchKernelGGL((k_gemm_q4k<WAVES_M, WAVES_N, TI, TJ, MINB>), dim3(tiles_n, tiles_m, splits),
                     dim3(256), 0, stream, w, x, y, m, n, k, per, splits > 1 ? 1 : 0);
  return hipGetLastError();
}


// ------------------------------------------------------------ large tiles
// 256 x 128 output tiles for large N at M >= 256 (each weight tile is then
// dequantized M/256 times instead of M/128 times):
//   * 8 waves, 4 (M) x 2 (N), 64 x 64 outputs each as 2 x 2 accumulators of
//     v_mfma_f32_32x32x16_bf16; two waves per SIMD, so one wave's LDS fragment
//     reads overlap the other's MFMAs.
//   * all global -> LDS traffic is direct (global_load_lds_dwordx4, no VGPR
//     staging): X through a 3-slot ring, the raw 16-byte header and 32 quant
//     bytes of each weight row through a 3-slot ring one step further ahead.
//     The copies are issued from inline assembly so the compiler neither
//     tracks nor waits for them; the waits are explicit: at the end of step s
//     the copies issued at step s-1 have landed (every wave issues exactly
//     kXCopies + 1 copies per step), then one barrier.
//   * the raw tile of step s+1 is dequantized (bf16, round to nearest even of
//     the exact fp32 weight) into one of two bf16 LDS tiles during step s.
//   * LDS rows are 128 bytes with the 16-byte chunks XOR-swizzled by row, so
//     the 32 rows a fragment read touches hit distinct banks.
//   * each workgroup starts its K loop at a different step: X rows are 8 KiB
//     apart, and workgroups walking K in lockstep would all hit the same L2
//     channel.
//   * when the tile grid allows, workgroup b (XCD b % 8) takes one M-tile
//     per group of XCDs, so each XCD's L2 holds one 2 MiB slice of X.
constexpr int kLBM = 256, kLBN = 128;
constexpr int kXCopies = kLBM * 128 / 1024 / 8;  // X copies (1 KiB each) per wave per step
constexpr int kLXSlot = kLBM * 128;              // bytes per X slot
constexpr int kLRSlot = kLBN * 64;               // bytes per raw-weight slot (64 B per row)
constexpr int kLBSlot = kLBN * 128;              // bytes per bf16 weight slot
constexpr int kLRot = 7;                         // K start step = blockIdx * 7 mod steps

__device__ __forceinline__ int swz(int r) { return ((r & 15) >> 1) ^ ((r & 1) << 2); }

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p));
}

// One 16-byte-per-lane global -> LDS copy: lane i's 16 bytes go to
// lds_uniform + 16 i.  M0 is saved and restored around the copy.
__device__ __forceinline__ void copy16_to_lds(const void* g, uint32_t lds_uniform) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(lds_uniform)
      : "memory");
}

__global__ __launch_bounds__(512, 1) void k_gemm_q4k_256x128(const uint8_t* __restrict__ w,
                                                             const uint16_t* __restrict__ x,
                                                             float* __restrict__ y, int m, int n,
                                                             int k, int tiles_m, int tiles_n,
                                                             int xcd_map) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[3 * kLXSlot + 3 * kLRSlot + 2 * kLBSlot];
  uint8_t* const xs = smem;
  uint8_t* const rs = smem + 3 * kLXSlot;
  uint8_t* const bs = smem + 3 * kLXSlot + 3 * kLRSlot;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int half = lane >> 5;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  int tm, tn;
  if (xcd_map) {
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int per_m = 8 / tiles_m;
    tm = xcd / per_m;
    tn = (xcd % per_m) * (tiles_n / per_m) + slot;
  } else {
    tm = blockIdx.x % tiles_m;
    tn = blockIdx.x / tiles_m;
  }
  const int m0 = tm * kLBM, n0 = tn * kLBN;
  const int kb_count = k >> 8;
  const int steps = k >> 6;
  const int rot = (static_cast<int>(blockIdx.x) * kLRot) % steps;
  // Physical K step of logical step s (steps past the end repeat the last one).
  auto phys = [&](int s) {
    const int e = min(s, steps - 1) + rot;
    return e < steps ? e : e - steps;
  };

  // X copies: copy q of this wave fills tile rows 8 (wave kXCopies + q) .. +7,
  // lane -> (row, LDS chunk lane % 8) holding X chunk (lane % 8) ^ swz(row).
  const uint16_t* xsrc[kXCopies];
#pragma unroll
  for (int q = 0; q < kXCopies; ++q) {
    const int row = 8 * (wave * kXCopies + q) + (lane >> 3);
    const int c = (lane & 7) ^ swz(row);
    xsrc[q] = x + static_cast<size_t>(min(m0 + row, m - 1)) * k + 8 * c;
  }
  // Raw-weight copy: wave fills rows 16 wave .. +15, lane -> (row, part):
  // part 0 header, 1 and 2 the two 16-byte halves of the quant group, 3 a
  // second header read that pads the row to 64 bytes.
  const int wrow = 16 * wave + (lane >> 2);
  const int wpart = lane & 3;
  const uint8_t* wsrc = w + static_cast<size_t>(min(n0 + wrow, n - 1)) * kb_count * kBlockBytes;
  const uint32_t xs_l = lds_address(xs), rs_l = lds_address(rs);

  auto copy_x = [&](int s, int slot) {
    const int ps = phys(s);
#pragma unroll
    for (int q = 0; q < kXCopies; ++q)
      copy16_to_lds(xsrc[q] + static_cast<size_t>(ps) * kBK,
                    __builtin_amdgcn_readfirstlane(xs_l + slot * kLXSlot +
                                                   (wave * kXCopies + q) * 1024));
  };
  auto copy_w = [&](int s, int slot) {
    const int ps = phys(s);
    const int off = (wpart == 1 || wpart == 2) ? 16 + 32 * (ps & 3) + 16 * (wpart - 1) : 0;
    copy16_to_lds(wsrc + static_cast<size_t>(ps >> 2) * kBlockBytes + off,
                  __builtin_amdgcn_readfirstlane(rs_l + slot * kLRSlot + wave * 1024));
  };

  // Dequant role: thread t -> weight row t / 4, quarter t % 4 of the quant
  // group (8 bytes: 8 low-nibble and 8 high-nibble weights).
  const int drow = t >> 2, dq = t & 3;
  auto read_raw = [&](int slot, uint4& hd, uint2& qv) {
    const uint8_t* rp = rs + slot * kLRSlot + drow * 64;
    hd = *reinterpret_cast<const uint4*>(rp);
    qv = *reinterpret_cast<const uint2*>(rp + 16 + 8 * dq);
  };
  auto dequant = [&](int s, const uint4& hd, const uint2& qv, int slot) {
    const GroupScales sc = group_scales(hd, phys(s) & 3);
    float lo[8], hi[8];
    dequant_dword(qv.x, sc, lo, hi);
    dequant_dword(qv.y, sc, lo + 4, hi + 4);
    uint8_t* rowp = bs + slot * kLBSlot + drow * 128;
    const int f = swz(drow);
    *reinterpret_cast<uint4*>(rowp + ((dq ^ f) << 4)) =
        make_uint4(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]),
                   pack_bf16x2(lo[4], lo[5]), pack_bf16x2(lo[6], lo[7]));
    *reinterpret_cast<uint4*>(rowp + (((4 + dq) ^ f) << 4)) =
        make_uint4(pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3]),
                   pack_bf16x2(hi[4], hi[5]), pack_bf16x2(hi[6], hi[7]));
  };

  f16x_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // A/B fragment of a K16 slice kk: lane -> row lane % 32, 16-byte chunk 2 kk + lane / 32.
  auto mfma_step = [&](int xslot, int bslot) {
    const uint8_t* xb = xs + xslot * kLXSlot;
    const uint8_t* wb = bs + bslot * kLBSlot;
    bf16x8_t af[4][2], bf[4][2];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int c = 2 * kk + half;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + 32 * i + (lane & 31);
        af[kk][i] = *reinterpret_cast<const bf16x8_t*>(xb + r * 128 + ((c ^ swz(r)) << 4));
        const int rn = wn * 64 + 32 * i + (lane & 31);
        bf[kk][i] = *reinterpret_cast<const bf16x8_t*>(wb + rn * 128 + ((c ^ swz(rn)) << 4));
      }
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk][i], bf[kk][j], acc[i][j], 0, 0, 0);
  };

  // Prologue: raw W(0), X(0), raw W(1), X(1), raw W(2) issued; W(0), X(0),
  // W(1) must land (X(1) and W(2): kXCopies + 1 copies may remain).
  static_assert(kXCopies + 1 == 5, "the explicit waits below count 5 copies per step");
  copy_w(0, 0);
  copy_x(0, 0);
  copy_w(1, 1);
  copy_x(1, 1);
  copy_w(2, 2);
  asm volatile("s_waitcnt vmcnt(5)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  {
    uint4 hd;
    uint2 qv;
    read_raw(0, hd, qv);
    dequant(0, hd, qv, 0);
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  // Step s: X slot s % 3, raw slot (s + 1) % 3, bf16 slot s % 2.
  int xa = 0, ra = 1, ba = 0;
  for (int s = 0; s < steps; ++s) {
    copy_x(s + 2, xa == 0 ? 2 : xa - 1);  // slot (s + 2) % 3, last read at step s - 1
    copy_w(s + 3, ra == 0 ? 2 : ra - 1);  // slot (s + 3) % 3, last read at step s - 1
    uint4 hd;
    uint2 qv;
    read_raw(ra, hd, qv);
    __builtin_amdgcn_sched_barrier(0);
    mfma_step(xa, ba);
    if (s + 1 < steps) dequant(s + 1, hd, qv, ba ^ 1);
    __builtin_amdgcn_sched_barrier(0);
    // copies of step s - 1 (X(s + 1), raw W(s + 2)) landed; LDS writes done
    asm volatile("s_waitcnt vmcnt(5)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    xa = xa == 2 ? 0 : xa + 1;
    ra = ra == 2 ? 0 : ra + 1;
    ba ^= 1;
  }
  // No copy into this workgroup's LDS may outlive it.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn * 64 + 32 * j + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 64 + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
        if (row < m && col < n) y[static_cast<size_t>(row) * n + col] = acc[i][j][r];
      }
    }
  }
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
    // Small batch: one 32-row slice, the four waves split the 128 weight rows.
    return launch<1, 4, 1, 1, 2>(w, x, y, mi, ni, ki, splits_for(tiles_n, steps), stream);
  }
  const int big_m = (mi + kLBM - 1) / kLBM, big_n = (ni + kLBN - 1) / kLBN;
  if (mi >= kLBM && big_m * big_n >= kGemmBigTiles) {
    // Enough 256 x 128 tiles to fill most CUs without splitting K.
    const bool xcd = 8 % big_m == 0 && big_n % (8 / big_m) == 0 && (big_m * big_n) % 8 == 0;
    hipLaunchKernelGGL(k_gemm_q4k_256x128, dim3(big_m * big_n), dim3(512), 0, stream, w, x, y,
                       mi, ni, ki, big_m, big_n, xcd ? 1 : 0);
    return hipGetLastError();
  }
  // 128 x 128 tiles, two workgroups per CU.
  const int tiles = ((mi + 127) / 128) * tiles_n;
  return launch<4, 1, 1, 4, 2>(w, x, y, mi, ni, ki, splits_for(tiles, steps), stream);
}

}  // namespace q4k
