// q4k_device.h -- gfx950 device routines that decode Q4_K super-blocks.
//
// Shared by every kernel of libq4k (GEMV, gate/up SwiGLU, GEMM tile fill,
// diagnostic dequant) so that all of them read the format the same way.
//
// Format (Q4_K as read by the library; the pages -- "Writing an ESIMD Fused
// Kernel From Reverse-Engineered Assembly", "Getting Q4_K Right" -- name the
// super-block, its 6-bit sub-block scales and mins and a quant-to-weight
// "y-offset mapping", but print no layout):
//   144 bytes = 16-byte header + 128 quant bytes, 256 weights.
//   header dword 0: d (fp16, bits 0..15), dmin (fp16, bits 16..31)
//   header dwords 1..3: scale bytes s[0..11]
//   quant group g (bytes 32g .. 32g+31): low nibble of byte 32g+r is weight
//   64g+r (sub-block 2g), high nibble is weight 64g+32+r (sub-block 2g+1).
//   w = d*sc[j]*q - dmin*mn[j].
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4k {

constexpr int kQK = 256;          // weights per super-block
constexpr int kBlockBytes = 144;  // bytes per Q4_K super-block

// Q5_K (the 5-bit sibling; "CPU kernel parity ..." PR page: k4 and k5 share
// one fused form; the layout is the GGUF reading, the pages print none):
//   176 bytes = the Q4_K header (16 bytes), 32 high-bit bytes qh, then the
//   128 Q4_K nibble bytes.  Weight 64g + r takes bit (2g + [r >= 32]) of
//   qh[r mod 32] as its fifth bit: q = nibble + 16 * bit.
constexpr int kQ5BlockBytes = 176;
constexpr int kQ5HighOffset = 16;   // qh[32]
constexpr int kQ5QuantOffset = 48;  // qs[128]

template <int FMT>
constexpr int block_bytes() {
  return FMT == 5 ? kQ5BlockBytes : kBlockBytes;
}

typedef float f2_t __attribute__((ext_vector_type(2)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// A byte 0000qqqq read as an OCP fp8 e4m3 value is q * 2^-9 exactly: codes
// 0..7 are the subnormals q * 2^-9 and codes 8..15 are (1 + (q-8)/8) * 2^-6
// = q * 2^-9.  gfx950 converts two such bytes to fp32 in one instruction, so
// nibbles are widened with the scale 2^-9 folded into the sub-block scale.
constexpr float kNibbleUnscale = 512.0f;

__device__ __forceinline__ f2_t fp8x2_lo(uint32_t v) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(v), false);
}
__device__ __forceinline__ f2_t fp8x2_hi(uint32_t v) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(v), true);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

// Scales of the two sub-blocks that quant group g feeds: 2g (low nibbles) and
// 2g+1 (high nibbles).  a = d*sc*2^9 multiplies an fp8-widened nibble, b =
// dmin*mn is subtracted.  All four products are exact in fp32 (an fp16 value
// times a 6-bit integer, times a power of two).
struct GroupScales {
  float a_lo, a_hi, b_lo, b_hi;
};

__device__ __forceinline__ GroupScales group_scales(uint4 h, int g) {
  // Per-byte 6-bit fields: bytes 0..3 of each word are sub-blocks 0..3 (lo)
  // or 4..7 (hi).
  const uint32_t sc_lo = h.y & 0x3F3F3F3Fu;
  const uint32_t mn_lo = h.z & 0x3F3F3F3Fu;
  const uint32_t sc_hi = (h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u);
  const uint32_t mn_hi = ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u);
  const int sh = (g & 1) * 16;
  const uint32_t sc = (g < 2 ? sc_lo : sc_hi) >> sh;
  const uint32_t mn = (g < 2 ? mn_lo : mn_hi) >> sh;
  const float d = half_bits_to_float(h.x & 0xFFFFu) * kNibbleUnscale;
  const float dmin = half_bits_to_float(h.x >> 16);
  GroupScales s;
  s.a_lo = d * static_cast<float>(sc & 0xFFu);
  s.a_hi = d * static_cast<float>((sc >> 8) & 0xFFu);
  s.b_lo = dmin * static_cast<float>(mn & 0xFFu);
  s.b_hi = dmin * static_cast<float>((mn >> 8) & 0xFFu);
  return s;
}

// Dequantize one quant dword (4 bytes = 4 low-nibble weights of sub-block 2g
// and 4 high-nibble weights of sub-block 2g+1) to fp32.  fma(a, q*2^-9, -b)
// rounds the exact d*sc*q - dmin*mn once, so the result is bit-identical to
// any correctly rounded evaluation.
__device__ __forceinline__ void dequant_dword(uint32_t v, const GroupScales& s, float lo[4],
                                              float hi[4]) {
  const uint32_t l = v & 0x0F0F0F0Fu;
  const uint32_t h = (v >> 4) & 0x0F0F0F0Fu;
  const f2_t l01 = fp8x2_lo(l), l23 = fp8x2_hi(l);
  const f2_t h01 = fp8x2_lo(h), h23 = fp8x2_hi(h);
  lo[0] = __builtin_fmaf(s.a_lo, l01.x, -s.b_lo);
  lo[1] = __builtin_fmaf(s.a_lo, l01.y, -s.b_lo);
  lo[2] = __builtin_fmaf(s.a_lo, l23.x, -s.b_lo);
  lo[3] = __builtin_fmaf(s.a_lo, l23.y, -s.b_lo);
  hi[0] = __builtin_fmaf(s.a_hi, h01.x, -s.b_hi);
  hi[1] = __builtin_fmaf(s.a_hi, h01.y, -s.b_hi);
  hi[2] = __builtin_fmaf(s.a_hi, h23.x, -s.b_hi);
  hi[3] = __builtin_fmaf(s.a_hi, h23.y, -s.b_hi);
}

// Q5_K: the four 5-bit quants of one quant dword's low (shift 0) or high
// (shift 4) nibbles, as bytes: nibbles plus the fifth bits, bit `hb` of each
// byte of the matching high-bit dword (hb = 2g for low nibbles, 2g + 1 for
// high ones).
__device__ __forceinline__ uint32_t q5_bytes(uint32_t v, uint32_t h, int shift, int hb) {
  return ((v >> shift) & 0x0F0F0F0Fu) | (((h >> hb) & 0x01010101u) << 4);
}

// Byte i of v as an exact float (one v_cvt_f32_ubyte<i>).
__device__ __forceinline__ float ubyte_f32(uint32_t v, int i) {
  return static_cast<float>((v >> (8 * i)) & 0xFFu);
}

// Round two fp32 values to bf16 (nearest even, v_cvt_pk_bf16_f32) and pack
// them: first value in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f2_t v = {a, b};
  const bf16x2_t r = __builtin_convertvector(v, bf16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}

// 8 weights as bf16: the nibbles at bit `shift` (0: low, 4: high) of the 8
// quant bytes in d0, d1 (byte order), each fma(a, q*2^-9, -b) rounded to
// nearest even, packed in pairs (first weight in the low half).  This is the
// MFMA operand routine of the GEMM kernels.
__device__ __forceinline__ bf16x8_t dequant8_bf16(uint32_t d0, uint32_t d1, int shift, float a,
                                                  float b) {
  const uint32_t l0 = (d0 >> shift) & 0x0F0F0F0Fu;
  const uint32_t l1 = (d1 >> shift) & 0x0F0F0F0Fu;
  const f2_t p0 = fp8x2_lo(l0), p1 = fp8x2_hi(l0), p2 = fp8x2_lo(l1), p3 = fp8x2_hi(l1);
  return __builtin_bit_cast(
      bf16x8_t,
      make_uint4(pack_bf16x2(__builtin_fmaf(a, p0.x, -b), __builtin_fmaf(a, p0.y, -b)),
                 pack_bf16x2(__builtin_fmaf(a, p1.x, -b), __builtin_fmaf(a, p1.y, -b)),
                 pack_bf16x2(__builtin_fmaf(a, p2.x, -b), __builtin_fmaf(a, p2.y, -b)),
                 pack_bf16x2(__builtin_fmaf(a, p3.x, -b), __builtin_fmaf(a, p3.y, -b))));
}

// Dequantize 16 quant bytes of group g (one 16-byte load) to bf16 through
// dequant8_bf16: lo8[0..7] are the 16 low-nibble weights (sub-block 2g) as 8
// packed pairs, hi8[0..7] the 16 high-nibble weights (sub-block 2g+1).  This
// is the bf16 diagnostic export and the tile fill of the split-K GEMM.
__device__ __forceinline__ void dequant16_bf16(uint4 q, const GroupScales& s, uint32_t lo8[8],
                                               uint32_t hi8[8]) {
  const uint4 l0 = __builtin_bit_cast(uint4, dequant8_bf16(q.x, q.y, 0, s.a_lo, s.b_lo));
  const uint4 l1 = __builtin_bit_cast(uint4, dequant8_bf16(q.z, q.w, 0, s.a_lo, s.b_lo));
  const uint4 h0 = __builtin_bit_cast(uint4, dequant8_bf16(q.x, q.y, 4, s.a_hi, s.b_hi));
  const uint4 h1 = __builtin_bit_cast(uint4, dequant8_bf16(q.z, q.w, 4, s.a_hi, s.b_hi));
  lo8[0] = l0.x; lo8[1] = l0.y; lo8[2] = l0.z; lo8[3] = l0.w;
  lo8[4] = l1.x; lo8[5] = l1.y; lo8[6] = l1.z; lo8[7] = l1.w;
  hi8[0] = h0.x; hi8[1] = h0.y; hi8[2] = h0.z; hi8[3] = h0.w;
  hi8[4] = h1.x; hi8[5] = h1.y; hi8[6] = h1.z; hi8[7] = h1.w;
}

// Q5_K: 8 weights as bf16 from the 5-bit quant bytes of two dwords (q5_bytes),
// each fma(a5, q, -b) with a5 = d*sc (no 2^9: the bytes are widened exactly by
// v_cvt_f32_ubyte), rounded to nearest even, packed in pairs.
__device__ __forceinline__ uint4 dequant8_bf16_q5(uint32_t q0, uint32_t q1, float a5, float b) {
  return make_uint4(pack_bf16x2(__builtin_fmaf(a5, ubyte_f32(q0, 0), -b),
                                __builtin_fmaf(a5, ubyte_f32(q0, 1), -b)),
                    pack_bf16x2(__builtin_fmaf(a5, ubyte_f32(q0, 2), -b),
                                __builtin_fmaf(a5, ubyte_f32(q0, 3), -b)),
                    pack_bf16x2(__builtin_fmaf(a5, ubyte_f32(q1, 0), -b),
                                __builtin_fmaf(a5, ubyte_f32(q1, 1), -b)),
                    pack_bf16x2(__builtin_fmaf(a5, ubyte_f32(q1, 2), -b),
                                __builtin_fmaf(a5, ubyte_f32(q1, 3), -b)));
}

// Q5_K: dequant16_bf16 for 16 quant bytes of group g with the 16 high-bit
// bytes of the same weights (qh[16hh ..] for quant bytes 32g + 16hh ..); s.a_*
// must already be d*sc (without the 2^9).
__device__ __forceinline__ void dequant16_bf16_q5(uint4 q, uint4 qh, const GroupScales& s, int g,
                                                  uint32_t lo8[8], uint32_t hi8[8]) {
  const uint4 l0 = dequant8_bf16_q5(q5_bytes(q.x, qh.x, 0, 2 * g), q5_bytes(q.y, qh.y, 0, 2 * g),
                                    s.a_lo, s.b_lo);
  const uint4 l1 = dequant8_bf16_q5(q5_bytes(q.z, qh.z, 0, 2 * g), q5_bytes(q.w, qh.w, 0, 2 * g),
                                    s.a_lo, s.b_lo);
  const uint4 h0 = dequant8_bf16_q5(q5_bytes(q.x, qh.x, 4, 2 * g + 1),
                                    q5_bytes(q.y, qh.y, 4, 2 * g + 1), s.a_hi, s.b_hi);
  const uint4 h1 = dequant8_bf16_q5(q5_bytes(q.z, qh.z, 4, 2 * g + 1),
                                    q5_bytes(q.w, qh.w, 4, 2 * g + 1), s.a_hi, s.b_hi);
  lo8[0] = l0.x; lo8[1] = l0.y; lo8[2] = l0.z; lo8[3] = l0.w;
  lo8[4] = l1.x; lo8[5] = l1.y; lo8[6] = l1.z; lo8[7] = l1.w;
  hi8[0] = h0.x; hi8[1] = h0.y; hi8[2] = h0.z; hi8[3] = h0.w;
  hi8[4] = h1.x; hi8[5] = h1.y; hi8[6] = h1.z; hi8[7] = h1.w;
}

__device__ __forceinline__ uint4 load16(const uint8_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// Sum of a float over the 64 lanes of a wave (every lane gets the total; all
// 64 lanes must be active).  Within a row of 16 lanes: DPP quad_perm xor-1 and
// xor-2, then row_ror 4 and 8; across the four rows: two DPP row broadcasts,
// then lane 63's total is read into every lane (the two lane swizzles through
// the LDS crossbar this replaces cost two LDS round trips and their lane
// arithmetic per sum).
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl,
                                                               kRowMask, 0xF, false));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
  v += dpp_mov<0x124>(v);  // row_ror 4
  v += dpp_mov<0x128>(v);  // row_ror 8: every lane holds its row's sum
  v += dpp_mov<0x142, 0xA>(v);  // row_bcast 15: rows 1 and 3 add the last lane of rows 0 and 2
  v += dpp_mov<0x143, 0xC>(v);  // row_bcast 31: rows 2 and 3 add lane 31 (rows 0 + 1)
  // Lane 63 holds (row 3 + row 2) + (row 1 + row 0); every lane returns it.
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

}  // namespace q4k
