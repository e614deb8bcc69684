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

// A unit's raw bytes as loaded: four 8-byte fields, each as the aligned dwords
// that hold it (a third dword only when the block starts 2 bytes past a dword
// boundary, s = 2), and d.
struct Q6Raw {
  uint32_t f[4][3];  // ql low half, ql high half, qh, scales of the half
  uint32_t d;
  uint32_t s;
};

__device__ __forceinline__ void load_field(const uint8_t* p, uint32_t s, uint32_t (&f)[3]) {
  const uint32_t* a = reinterpret_cast<const uint32_t*>(p - s);
  f[0] = a[0];
  f[1] = a[1];
  f[2] = 0u;
  if (s) f[2] = a[2];
}

__device__ __forceinline__ Q6Raw load_raw(const uint8_t* blk, int h, int c) {
  Q6Raw r;
  r.s = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(blk) & 3u);
  load_field(blk + 64 * h + 8 * c, r.s, r.f[0]);
  load_field(blk + 64 * h + 32 + 8 * c, r.s, r.f[1]);
  load_field(blk + 128 + 32 * h + 8 * c, r.s, r.f[2]);
  load_field(blk + 192 + 8 * h, r.s, r.f[3]);
  r.d = *reinterpret_cast<const uint16_t*>(blk + 208);
  return r;
}

// The fields of one unit: quants q[j][e / 4] (four 6-bit values per dword,
// weight e in byte e % 4), the four scales d * sc (exact in fp32).
struct Q6Unit {
  uint32_t q[4][2];
  float dsc[4];
};

__device__ __forceinline__ Q6Unit decode_unit(const Q6Raw& r, int c) {
  // v_alignbyte_b32(hi, lo, n) = the 64-bit {hi, lo} shifted right by n bytes (n = 0..3)
  uint32_t v[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i][0] = __builtin_amdgcn_alignbyte(r.f[i][1], r.f[i][0], r.s);
    v[i][1] = __builtin_amdgcn_alignbyte(r.f[i][2], r.f[i][1], r.s);
  }
  Q6Unit u;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const uint32_t L = v[0][e], H = v[1][e], Q = v[2][e];
    u.q[0][e] = (L & 0x0F0F0F0Fu) | ((Q << 4) & 0x30303030u);
    u.q[1][e] = (H & 0x0F0F0F0Fu) | ((Q << 2) & 0x30303030u);
    u.q[2][e] = ((L >> 4) & 0x0F0F0F0Fu) | (Q & 0x30303030u);
    u.q[3][e] = ((H >> 4) & 0x0F0F0F0Fu) | ((Q >> 2) & 0x30303030u);
  }
  const float d = half_bits_to_float(r.d);
  const int cb = c >> 1;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int b = 2 * j + cb;  // scale byte within the half: sub-block 8h + 2j + c/2
    const uint32_t word = b < 4 ? v[3][0] : v[3][1];
    const int sv = static_cast<int>(static_cast<int8_t>((word >> (8 * (b & 3))) & 0xFFu));
    u.dsc[j] = d * static_cast<float>(sv);
  }
  return u;
}

__device__ __forceinline__ Q6Unit load_unit(const uint8_t* blk, int h, int c) {
  return decode_unit(load_raw(blk, h, c), c);
}

// GEMV: a workgroup of 4 waves, 4 rows per wave; per 4096-wide chunk of x a
// lane owns units lane and lane + 64 (8 units per block).  The weight loads of
// the chunk are issued first, then x is staged, so the staging round trip
// overlaps the weight stream.
constexpr int kQ6UnitsPerLane = kQ6Chunk / 32 / 64;

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
    const int units = kc >> 5;             // 8 per block
    // Units past a short chunk's end re-read its last unit (not accumulated).
    Q6Raw raw[kQ6UnitsPerLane][kQ6RowsPerWave];
#pragma unroll
    for (int t = 0; t < kQ6UnitsPerLane; ++t) {
      const int u = min(lane + 64 * t, units - 1);
      const int bg = (c0 >> 8) + (u >> 3);
#pragma unroll
      for (int r = 0; r < kQ6RowsPerWave; ++r)
        raw[t][r] = load_raw(rows[r] + static_cast<size_t>(bg) * kQ6Bytes, (u >> 2) & 1, u & 3);
    }
    __syncthreads();  // the previous chunk's reads of xs are done
    for (int i = 4 * static_cast<int>(threadIdx.x); i < kc; i += 4 * 256)
      *reinterpret_cast<float4*>(xs + i) = *reinterpret_cast<const float4*>(x + c0 + i);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < kQ6UnitsPerLane; ++t) {
      const int u = lane + 64 * t;
      if (u >= units) continue;
      const int bl = u >> 3, h = (u >> 2) & 1, c = u & 3;
      float xv[4][8], s8[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float* p = xs + 256 * bl + 128 * h + 32 * j + 8 * c;
        const float4 a = *reinterpret_cast<const float4*>(p);
        const float4 b = *reinterpret_cast<const float4*>(p + 4);
        xv[j][0] = a.x; xv[j][1] = a.y; xv[j][2] = a.z; xv[j][3] = a.w;
        xv[j][4] = b.x; xv[j][5] = b.y; xv[j][6] = b.z; xv[j][7] = b.w;
        s8[j] = ((a.x + a.y) + (a.z + a.w)) + ((b.x + b.y) + (b.z + b.w));
      }
#pragma unroll
      for (int r = 0; r < kQ6RowsPerWave; ++r) {
        const Q6Unit wu = decode_unit(raw[t][r], c);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float dot = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) dot = fmaf(ubyte_f32(wu.q[j][e >> 2], e & 3), xv[j][e], dot);
          acc[r] = fmaf(wu.dsc[j], fmaf(-32.0f, s8[j], dot), acc[r]);
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
