// k_dequant.hip -- diagnostic export of a Q4_K matrix as fp32 or bf16.
//
// Runs the same device routines as the GEMV (group_scales, dequant_dword)
// and the GEMM tile fill (dequant16_bf16), so the bit-exact check of this
// export ("CPU kernel parity ..." PR page, "Validation": every variant
// bit-exact against the reference decode) covers what the other kernels
// compute.
//
// One thread per 16 quant bytes: (row, block, group g, half hh).  It writes
// the 16 low-nibble weights 64g+16hh.. and the 16 high-nibble weights
// 64g+32+16hh.. of its block.
#include <hip/hip_runtime.h>

#include "q4k_device.h"
#include "q4k_launch.h"

namespace q4k {
namespace {

template <bool BF16>
__global__ __launch_bounds__(256) void k_dequant_q4k(const uint8_t* __restrict__ w,
                                                     void* __restrict__ out, size_t chunks) {
  const size_t t = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (t >= chunks) return;
  const int hh = static_cast<int>(t & 1);
  const int g = static_cast<int>((t >> 1) & 3);
  const size_t blk = t >> 3;  // row * (k/256) + block
  const uint8_t* p = w + blk * kBlockBytes;
  const uint4 hd = load16(p);
  const uint4 q = load16(p + 16 + 32 * g + 16 * hh);
  const GroupScales s = group_scales(hd, g);
  // Row-major [n, k]: weight (row, 256*block + i) is element blk*256 + i.
  const size_t base = blk * kQK + 64 * g + 16 * hh;
  if constexpr (BF16) {
    uint32_t lo8[8], hi8[8];
    dequant16_bf16(q, s, lo8, hi8);
    uint4* o = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + base);
    o[0] = make_uint4(lo8[0], lo8[1], lo8[2], lo8[3]);
    o[1] = make_uint4(lo8[4], lo8[5], lo8[6], lo8[7]);
    uint4* o2 = reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + base + 32);
    o2[0] = make_uint4(hi8[0], hi8[1], hi8[2], hi8[3]);
    o2[1] = make_uint4(hi8[4], hi8[5], hi8[6], hi8[7]);
  } else {
    float* o = static_cast<float*>(out) + base;
    const uint32_t v[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float lo[4], hi[4];
      dequant_dword(v[i], s, lo, hi);
      *reinterpret_cast<f4_t*>(o + 4 * i) = f4_t{lo[0], lo[1], lo[2], lo[3]};
      *reinterpret_cast<f4_t*>(o + 32 + 4 * i) = f4_t{hi[0], hi[1], hi[2], hi[3]};
    }
  }
}

template <bool BF16>
hipError_t launch(const uint8_t* w, void* out, int64_t n, int64_t k, hipStream_t stream) {
  const size_t chunks = static_cast<size_t>(n) * static_cast<size_t>(k / kQK) * 8;
  const size_t grid = (chunks + 255) / 256;
  hipLaunchKernelGGL((k_dequant_q4k<BF16>), dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                     stream, w, out, chunks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dequant_f32(const uint8_t* w, float* out, int64_t n, int64_t k,
                              hipStream_t stream) {
  return launch<false>(w, out, n, k, stream);
}

hipError_t launch_dequant_bf16(const uint8_t* w, uint16_t* out, int64_t n, int64_t k,
                               hipStream_t stream) {
  return launch<true>(w, out, n, k, stream);
}

}  // namespace q4k
