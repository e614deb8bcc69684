// k_q6k.hip -- Q6_K (the 6-bit k-quant): decode GEMV and the dequant export.
//
// Format (the daScript PR page "CPU kernel parity: decode and tile kernels at
// llama.cpp speed ..." names "k6", its high-bit plane and its per-sub-block
// scales; the layout is the GGUF reading, the pages print none):
//   210 bytes per 256 weights: ql[128] at 0, qh[64] at 128, signed 8-bit
//   scales sc[16] at 192, fp16 d at 208.  Weight 128h + 32j + l: low nibble
//   (j < 2) or high nibble (j >= 2) of ql[64h + 32(j mod 2) + l], bits 2j and
//   2j+1 of qh[32h + l] on top; w = d * sc[i / 16] * (q - 32).
//
// Design for gfx950:
//   * A unit is (block, h, c): the 32 weights 128h + 32j + 8c + e (j = 0..3,
//     e = 0..7).  It reads 8 bytes of each nibble half (ql[64h + 8c ..] and
//     ql[64h + 32 + 8c ..]), 8 high-bit bytes (qh[32h + 8c ..]), the 8 scale
//     bytes of its half and d; four quants of one j come out of each pair of
//     dwords with two masks, a shift and an OR, in the bytes' order.
//   * Blocks are 210 bytes, so a block starts 0 or 2 bytes past a dword
//     boundary (the matrix itself is 16-byte aligned).  Every field read above
//     sits at a multiple of 4 inside the block: it is read as aligned dwords
//     from the dword boundary below it, plus one more dword when the block is
//     2 bytes off, and v_alignbyte shifts the bytes into place.  No read leaves
//     the block, and d is read with one 16-bit load.
//   * The scale of sub-block (j, c / 2) multiplies a sum of 8 weights: per unit
//     and j the GEMV forms dot = sum q x and s8 = sum x in fp32 and adds
//     (d sc) (dot - 32 s8) to its partial sum; the (q - 32) offset costs one
//     FMA per 8 weights.
//   * GEMV: a workgroup of 4 waves owns 16 consecutive rows (4 per wave); each
//     4096-wide chunk of x is staged once per workgroup in LDS and every lane
//     copies the 32 x values (and their 8-sums) of each of its units into
//     registers, reused for all four rows.  Batches run one x row per launch.
//   * Dequant export: one thread per unit, fp32 = (d sc) * (q - 32) (the exact
//     product rounded once: d sc is exact in fp32) or its bf16 (nearest even).
#include <hip/hip_runtime.h>

#include "q4k_device.h"
#include "q4k_launch.h"

namespace q4k {
namespace {

constexpr int kQ6Bytes = 210;
constexpr int kQ6Chunk = 4096;   // x elements staged per pass (16 KiB)
constexpr int kQ6RowsPerWave = 4;

// 8 bytes at address p, with s = p mod 4 in {0, 2}: aligned dword loads from
// p - s (a third one only when s = 2), shifted into place.
__device__ __forceinline__ uint2 load8_q6(const uint8_t* p, uint32_t s) {
  const uint32_t* a = reinterpret_cast<const uint32_t*>(p - s);
  const uint32_t a0 = a[0], a1 = a[1];
  uint32_t a2 = 0u;
  if (s) a2 = a[2];
  // v_alignbyte_b32(hi, lo, n) = the 64-bit {hi, lo} shifted right by n bytes (n = 0..3)
  return uint2{__builtin_amdgcn_alignbyte(a1, a0, s), __builtin_amdgcn_alignbyte(a2, a1, s)};
}

// The fields of one unit: quants q[j][e / 4] (four 6-bit values per dword,
// weight e in byte e % 4), the four scales d * sc (exact in fp32).
struct Q6Unit {
  uint32_t q[4][2];
  float dsc[4];
};

__device__ __forceinline__ Q6Unit load_unit(const uint8_t* blk, int h, int c) {
  const uint32_t s = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(blk) & 3u);
  const uint2 lo = load8_q6(blk + 64 * h + 8 * c, s);
  const uint2 hi = load8_q6(blk + 64 * h + 32 + 8 * c, s);
  const uint2 qh = load8_q6(blk + 128 + 32 * h + 8 * c, s);
  const uint2 sc = load8_q6(blk + 192 + 8 * h, s);
  const uint32_t dbits = *reinterpret_cast<const uint16_t*>(blk + 208);
  Q6Unit u;
  const uint32_t L[2] = {lo.x, lo.y}, H[2] = {hi.x, hi.y}, Q[2] = {qh.x, qh.y};
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    u.q[0][e] = (L[e] & 0x0F0F0F0Fu) | ((Q[e] << 4) & 0x30303030u);
    u.q[1][e] = (H[e] & 0x0F0F0F0Fu) | ((Q[e] << 2) & 0x30303030u);
    u.q[2][e] = ((L[e] >> 4) & 0x0F0F0F0Fu) | (Q[e] & 0x30303030u);
    u.q[3][e] = ((H[e] >> 4) & 0x0F0F0F0Fu) | ((Q[e] >> 2) & 0x30303030u);
  }
  const float d = half_bits_to_float(dbits);
  const int cb = c >> 1;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int b = 2 * j + cb;  // scale byte within the half: sub-block 8h + 2j + c/2
    const uint32_t word = b < 4 ? sc.x : sc.y;
    const int v = static_cast<int>(static_cast<int8_t>((word >> (8 * (b & 3))) & 0xFFu));
    u.dsc[j] = d * static_cast<float>(v);
  }
  return u;
}

// The 32 x values of a unit (x[j][e]) and their 8-sums.
struct Q6X {
  float x[4][8];
  float s8[4];
};

__global__ __launch_bounds__(256) void k_gemv_q6k(const uint8_t* __restrict__ w,
                                                  const float* __restrict__ x,
                                                  float* __restrict__ y, int n, int k) {
  __shared__ __attribute__((aligned(16))) float xs[kQ6Chunk];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row0 = (blockIdx.x * 4 + wave) * kQ6RowsPerWave;
  const int nb = k >> 8;
  const size_t row_bytes = static_cast<size_t>(nb) * kQ6Bytes;
  const uint8_t* rows[kQ6RowsPerWave];
#pragma unroll
  for (int r = 0; r < kQ6RowsPerWave; ++r)
    rows[r] = w + static_cast<size_t>(min(row0 + r, n - 1)) * row_bytes;
  float acc[kQ6RowsPerWave];
#pragma unroll
  for (int r = 0; r < kQ6RowsPerWave; ++r) acc[r] = 0.0f;

  for (int c0 = 0; c0 < k; c0 += kQ6Chunk) {
    const int kc = min(kQ6Chunk, k - c0);  // a multiple of 256
    __syncthreads();                       // the previous chunk's reads are done
    for (int i = 4 * static_cast<int>(threadIdx.x); i < kc; i += 4 * 256)
      *reinterpret_cast<float4*>(xs + i) = *reinterpret_cast<const float4*>(x + c0 + i);
    __syncthreads();
    const int units = kc >> 5;  // 8 per block
    for (int u = lane; u < units; u += 64) {
      const int bl = u >> 3, h = (u >> 2) & 1, c = u & 3;
      Q6X xv;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float* p = xs + 256 * bl + 128 * h + 32 * j + 8 * c;
        const float4 a = *reinterpret_cast<const float4*>(p);
        const float4 b = *reinterpret_cast<const float4*>(p + 4);
        xv.x[j][0] = a.x; xv.x[j][1] = a.y; xv.x[j][2] = a.z; xv.x[j][3] = a.w;
        xv.x[j][4] = b.x; xv.x[j][5] = b.y; xv.x[j][6] = b.z; xv.x[j][7] = b.w;
        xv.s8[j] = ((a.x + a.y) + (a.z + a.w)) + ((b.x + b.y) + (b.z + b.w));
      }
      const int bg = (c0 >> 8) + bl;  // block index within the row
      Q6Unit wu[kQ6RowsPerWave];
#pragma unroll
      for (int r = 0; r < kQ6RowsPerWave; ++r)
        wu[r] = load_unit(rows[r] + static_cast<size_t>(bg) * kQ6Bytes, h, c);
#pragma unroll
      for (int r = 0; r < kQ6RowsPerWave; ++r) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float dot = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) dot = fmaf(ubyte_f32(wu[r].q[j][e >> 2], e & 3), xv.x[j][e], dot);
          acc[r] = fmaf(wu[r].dsc[j], fmaf(-32.0f, xv.s8[j], dot), acc[r]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kQ6RowsPerWave; ++r) {
    const float v = wave_sum(acc[r]);
    if (lane == 0 && row0 + r < n) y[row0 + r] = v;
  }
}

// One thread per unit of the matrix (8 per block), rows of k/256 blocks.
template <bool BF16>
__global__ __launch_bounds__(256) void k_dequant_q6k(const uint8_t* __restrict__ w,
                                                     void* __restrict__ out, int64_t units) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= units) return;
  const int64_t g = t >> 3;  // global block index = row * nb + b
  const int h = static_cast<int>((t >> 2) & 1), c = static_cast<int>(t & 3);
  const Q6Unit u = load_unit(w + g * kQ6Bytes, h, c);
  // block g covers output elements 256 g .. 256 g + 255 of the row-major [n, k]
  const int64_t base = 256 * g + 128 * h + 8 * c;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      v[e] = u.dsc[j] * (ubyte_f32(u.q[j][e >> 2], e & 3) - 32.0f);
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

}  // namespace

hipError_t launch_q6k_gemv(const uint8_t* w, const float* x, float* y, int64_t m, int64_t n,
                           int64_t k, hipStream_t stream) {
  const int ni = static_cast<int>(n), ki = static_cast<int>(k);
  const int rows_per_wg = 4 * kQ6RowsPerWave;
  const dim3 grid(static_cast<unsigned>((ni + rows_per_wg - 1) / rows_per_wg));
  for (int64_t i = 0; i < m; ++i) {
    hipLaunchKernelGGL(k_gemv_q6k, grid, dim3(256), 0, stream, w, x + i * k, y + i * n, ni, ki);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_q6k_dequant_f32(const uint8_t* w, float* out, int64_t n, int64_t k,
                                  hipStream_t stream) {
  const int64_t units = n * (k / 256) * 8;
  hipLaunchKernelGGL((k_dequant_q6k<false>), dim3(static_cast<unsigned>((units + 255) / 256)),
                     dim3(256), 0, stream, w, out, units);
  return hipGetLastError();
}

hipError_t launch_q6k_dequant_bf16(const uint8_t* w, uint16_t* out, int64_t n, int64_t k,
                                   hipStream_t stream) {
  const int64_t units = n * (k / 256) * 8;
  hipLaunchKernelGGL((k_dequant_q6k<true>), dim3(static_cast<unsigned>((units + 255) / 256)),
                     dim3(256), 0, stream, w, out, units);
  return hipGetLastError();
}

}  // namespace q4k
