// lds_copy.h -- gfx950 building blocks shared by the LDS-staged GEMM kernels:
// direct global -> LDS copies, the XOR swizzle of 128-byte LDS rows, and the
// XCD-aware tile order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4k {

// 16-byte chunk position of a 128-byte LDS row r: chunk c of row r is stored
// at chunk c ^ swz(r).  Any 16 consecutive rows then put a given chunk in 16
// distinct 4-bank groups, so a ds_read_b128 of one chunk from 16 rows is
// conflict-free.
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

// Direct global -> LDS copy of 16 bytes per lane from sbase + voff (sbase
// uniform, in SGPRs; voff a per-lane 32-bit byte offset) to lds_uniform + 16
// lane.  M0 is saved and restored around the copy.
__device__ __forceinline__ void copy16_to_lds_so(uint32_t voff, const void* sbase,
                                                 uint32_t lds_uniform) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds_uniform)
      : "memory");
}

template <int N>
__device__ __forceinline__ void wait_copies() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most N copies of this wave are in flight, then barrier.
template <int N>
__device__ __forceinline__ void wait_copies_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Output tile of workgroup `bid`.  Workgroups are dealt to the eight XCDs in
// turn (XCD = bid mod 8), each with its own L2.  With xcd_gm = 0 the tiles run
// M-fastest.  Otherwise the tile grid is cut into gm x (8 / gm) blocks, one per
// XCD, so that an XCD's workgroups share their X rows and weight columns in its
// L2 instead of every XCD fetching all of W (needs tiles_m % gm == 0 and
// tiles_n % (8 / gm) == 0; the host picks gm).
__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int xcd_gm,
                                            int& tm, int& tn) {
  if (xcd_gm) {
    const int xcd = bid & 7, slot = bid >> 3;
    const int a = tiles_m / xcd_gm;  // M-tiles per XCD block
    tm = (xcd % xcd_gm) * a + slot % a;
    tn = (xcd / xcd_gm) * (tiles_n / (8 / xcd_gm)) + slot / a;
  } else {
    tm = bid % tiles_m;
    tn = bid / tiles_m;
  }
}


// Host side: the gm of tile_coords that minimizes the bytes an XCD fetches
// per step, m_cost per M-tile and n_cost per N-tile of its block (0 when no
// blocking divides the grid).
inline int xcd_blocking(int tiles_m, int tiles_n, long m_cost, long n_cost) {
  int best = 0;
  long best_cost = 0;
  for (int gm = 1; gm <= 8; gm *= 2) {
    const int gn = 8 / gm;
    if (tiles_m % gm != 0 || tiles_n % gn != 0) continue;
    const long cost = (tiles_m / gm) * m_cost + (tiles_n / gn) * n_cost;
    if (best == 0 || cost < best_cost) {
      best = gm;
      best_cost = cost;
    }
  }
  return best;
}

}  // namespace q4k
