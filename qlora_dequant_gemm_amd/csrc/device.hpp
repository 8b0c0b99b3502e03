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

// Per-block magnitude table in byte planes: entry j (0..7) = bf16(L[15-j] * s),
// the magnitudes largest first; low and high bytes in two dwords each.
struct MagTable {
  uint32_t lo0, lo1, hi0, hi1;
};

__device__ __forceinline__ MagTable make_table(const Codebook& cb, float s) {
  const uint32_t p0 = pack_bf16x2(cb.L[15] * s, cb.L[14] * s);
  const uint32_t p1 = pack_bf16x2(cb.L[13] * s, cb.L[12] * s);
  const uint32_t p2 = pack_bf16x2(cb.L[11] * s, cb.L[10] * s);
  const uint32_t p3 = pack_bf16x2(cb.L[9] * s, cb.L[8] * s);
  MagTable t;
  t.lo0 = perm(p1, p0, 0x06040200u);
  t.hi0 = perm(p1, p0, 0x07050301u);
  t.lo1 = perm(p3, p2, 0x06040200u);
  t.hi1 = perm(p3, p2, 0x07050301u);
  return t;
}

// v_bitop3_b32 with truth table kTT (bit 4a + 2b + c of kTT is the result for
// input bits a, b, c). Called by name because the compiler rewrites the masked
// forms below into sequences one or two operations longer.
template <int kTT>
__device__ __forceinline__ uint32_t bitop3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, kTT);
}
constexpr int kTTXorAnd = 0x28;      // (a ^ b) & c
constexpr int kTTOrAndNot = 0xF2;    // a | (~b & c)

// The byte planes of the 8 codes of one packed dword (element 2i in the low
// nibble of byte i): even elements (0 2 4 6) in loE/hiE, odd ones in loO/hiO.
// Code c maps to magnitude index c (c < 8) or 15 - c (c >= 8), i.e. c XOR 7b
// with b = bit 3 of c, masked to 3 bits, for all eight nibbles at once; the
// sign bit of the high byte is set where bit 3 of the code is clear.
struct Planes {
  uint32_t loE, hiE, loO, hiO;
};
__device__ __forceinline__ Planes lookup8(uint32_t d, const MagTable& t) {
  const uint32_t n8 = d & 0x88888888u;                   // bit 3 of every code
  const uint32_t f = n8 - (n8 >> 3);                     // 7 in every nibble with bit 3 set
  const uint32_t se = bitop3<kTTXorAnd>(d, f, 0x07070707u);
  const uint32_t so = bitop3<kTTXorAnd>(d, f, 0x70707070u) >> 4;
  Planes p;
  p.loE = perm(t.lo1, t.lo0, se);
  p.hiE = bitop3<kTTOrAndNot>(perm(t.hi1, t.hi0, se), d << 4, 0x80808080u);
  p.loO = perm(t.lo1, t.lo0, so);
  p.hiO = bitop3<kTTOrAndNot>(perm(t.hi1, t.hi0, so), d, 0x80808080u);
  return p;
}

// One packed dword -> 8 bf16 in natural order, as 4 dwords of bf16 pairs
// (21 VALU operations).
__device__ __forceinline__ u32x4 decode8(uint32_t d, const MagTable& t) {
  const Planes p = lookup8(d, t);
  // interleave even and odd elements per plane, then pair low and high bytes
  const uint32_t l03 = perm(p.loO, p.loE, 0x05010400u);
  const uint32_t l47 = perm(p.loO, p.loE, 0x07030602u);
  const uint32_t h03 = perm(p.hiO, p.hiE, 0x05010400u);
  const uint32_t h47 = perm(p.hiO, p.hiE, 0x07030602u);
  u32x4 r;
  r.x = perm(h03, l03, 0x05010400u);
  r.y = perm(h03, l03, 0x07030602u);
  r.z = perm(h47, l47, 0x05010400u);
  r.w = perm(h47, l47, 0x07030602u);
  return r;
}

// The same 8 bf16 in the order 0 2 | 4 6 | 1 3 | 5 7 (17 VALU operations):
// for contractions whose other operand is permuted the same way.
__device__ __forceinline__ u32x4 decode8_perm(uint32_t d, const MagTable& t) {
  const Planes p = lookup8(d, t);
  u32x4 r;
  r.x = perm(p.hiE, p.loE, 0x05010400u);
  r.y = perm(p.hiE, p.loE, 0x07030602u);
  r.z = perm(p.hiO, p.loO, 0x05010400u);
  r.w = perm(p.hiO, p.loO, 0x07030602u);
  return r;
}

// 8 consecutive bf16 (4 dwords, low half first) -> the order 0 2 | 4 6 | 1 3 | 5 7
__device__ __forceinline__ u32x4 perm8(const u32x4& v) {
  u32x4 r;
  r.x = perm(v.y, v.x, 0x05040100u);
  r.y = perm(v.w, v.z, 0x05040100u);
  r.z = perm(v.y, v.x, 0x07060302u);
  r.w = perm(v.w, v.z, 0x07060302u);
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
