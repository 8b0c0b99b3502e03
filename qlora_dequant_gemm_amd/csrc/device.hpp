// Device helpers shared by the gfx950 kernels: vector types, byte permutes,
// bf16 packing and the per-block NF4 -> bf16 decode.
//
// Dequantization ("A 65B fine-tune on the GPU you already have", figure 2:
// weights become bf16 block by block right before the multiply):
//   w' = bf16_rne(L[c] * s),  s = fp32(q * d)
// Every block of 64 weights shares s, so a block has only 16 possible outputs.
// Because the levels are exactly antisymmetric (L[7-i] == -L[8+i]) and both
// the fp32 product and round-to-nearest-even are sign-symmetric, the 8
// magnitudes |bf16(L[8+i] * s)| plus a sign bit give all 16. The magnitudes
// are kept as two byte planes of 8 bytes (low bytes, high bytes), so one
// v_perm_b32 looks up four codes at once in one plane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "codebook.hpp"

namespace qnf4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// Byte select from the 8 bytes {hi:lo}: selector byte 0-3 -> lo, 4-7 -> hi,
// 0x0C -> 0x00, 0x0D..0x0F -> 0xFF (v_perm_b32).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t p) { return __builtin_bit_cast(float, p << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t p) { return __builtin_bit_cast(float, p & 0xFFFF0000u); }

// Per-block magnitude table in byte planes: entry i = bf16(L[8+i] * s).
struct MagTable {
  uint32_t lo0, lo1, hi0, hi1;
};

__device__ __forceinline__ MagTable make_table(const Codebook& cb, float s) {
  const uint32_t p0 = pack_bf16x2(cb.L[8] * s, cb.L[9] * s);
  const uint32_t p1 = pack_bf16x2(cb.L[10] * s, cb.L[11] * s);
  const uint32_t p2 = pack_bf16x2(cb.L[12] * s, cb.L[13] * s);
  const uint32_t p3 = pack_bf16x2(cb.L[14] * s, cb.L[15] * s);
  MagTable t;
  t.lo0 = perm(p1, p0, 0x06040200u);
  t.hi0 = perm(p1, p0, 0x07050301u);
  t.lo1 = perm(p3, p2, 0x06040200u);
  t.hi1 = perm(p3, p2, 0x07050301u);
  return t;
}

// Four codes, one per byte (values 0..15 in bits 0-3; bit 3 also given by
// `pos` = 1 per byte when the code is >= 8): low and high bf16 byte planes.
//   code >= 8: magnitude index code-8 = code ^ 8, positive
//   code <  8: magnitude index 7-code = code ^ 7, negative
__device__ __forceinline__ void lookup4(uint32_t codes, uint32_t pos, const MagTable& t,
                                        uint32_t& lo, uint32_t& hi) {
  const uint32_t mi = (codes ^ (pos + 0x07070707u)) & 0x07070707u;
  lo = perm(t.lo1, t.lo0, mi);
  hi = perm(t.hi1, t.hi0, mi) ^ ((pos ^ 0x01010101u) << 7);
}

// One packed dword (8 codes, element 2i in the low nibble of byte i) ->
// 8 bf16 in natural order, as 4 dwords of bf16 pairs.
__device__ __forceinline__ u32x4 decode8(uint32_t d, const MagTable& t) {
  uint32_t loE, hiE, loO, hiO;
  lookup4(d, (d >> 3) & 0x01010101u, t, loE, hiE);          // even elements
  lookup4(d >> 4, (d >> 7) & 0x01010101u, t, loO, hiO);     // odd elements
  // interleave: [lo e0, lo e1, lo e2, lo e3] etc., then lo/hi into pairs
  const uint32_t l03 = perm(loO, loE, 0x05010400u);
  const uint32_t l47 = perm(loO, loE, 0x07030602u);
  const uint32_t h03 = perm(hiO, hiE, 0x05010400u);
  const uint32_t h47 = perm(hiO, hiE, 0x07030602u);
  u32x4 r;
  r.x = perm(h03, l03, 0x05010400u);
  r.y = perm(h03, l03, 0x07030602u);
  r.z = perm(h47, l47, 0x05010400u);
  r.w = perm(h47, l47, 0x07030602u);
  return r;
}

// Block scale s = fp32(q * d) of the double-quantized constants.
__device__ __forceinline__ float block_scale(int8_t q, float d) {
  return static_cast<float>(q) * d;
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

}  // namespace qnf4
