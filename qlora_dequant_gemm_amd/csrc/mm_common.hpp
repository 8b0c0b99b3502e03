// Device helpers shared by the matmul kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"
#include "kernels.hpp"

namespace qnf4 {

typedef __attribute__((address_space(3))) short lds_short;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ uint16_t bf16_bits(float v) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}

// 8 bf16 of `row` starting at col0, zero past len; one 16-byte load when the
// whole run is in range and rows are 16-byte aligned.
__device__ __forceinline__ u32x4 load_row8(const uint16_t* row, int64_t col0, int64_t len, bool vec_ok) {
  if (vec_ok && col0 + 8 <= len) return ld16(row + col0);
  uint32_t v[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int64_t c = col0 + e;
    const uint32_t b = (c < len) ? static_cast<uint32_t>(row[c]) : 0u;
    v[e >> 1] |= b << (16 * (e & 1));
  }
  return u32x4{v[0], v[1], v[2], v[3]};
}

__device__ __forceinline__ int64_t imin(int64_t a, int64_t b) { return a < b ? a : b; }

__device__ __forceinline__ s16x4 ds_read_tr(const u32x4* base, int elem_off) {
  // generic -> LDS address space (the pointer always refers to __shared__ memory)
  lds_short* p = (lds_short*)(const_cast<short*>(reinterpret_cast<const short*>(base))) + elem_off;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
}

typedef __attribute__((address_space(3))) void lds_void;

// Workgroup barrier without a fence: the wait for global loads in flight that
// __syncthreads' fence implies is left out (prefetches stay in flight across
// it); the caller waits for its own LDS writes and buffer-to-LDS loads first.
// The compiler sees the asm as touching memory, but may still move accesses
// to a __shared__ array whose address never escapes across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }
// The same after this wave's LDS operations are done, with the kernel's
// __shared__ arrays named as operands, so that no access to them moves across.
template <typename A, typename B, typename C, typename D>
__device__ __forceinline__ void lds_barrier_on(A* a, B* b, C* c, D* d) {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::"s"(a), "s"(b), "s"(c), "s"(d) : "memory");
}
template <typename A, typename B, typename C, typename D, typename E, typename F>
__device__ __forceinline__ void lds_barrier_on(A* a, B* b, C* c, D* d, E* e, F* f) {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::"s"(a), "s"(b), "s"(c), "s"(d), "s"(e), "s"(f) : "memory");
}

// s_waitcnt vmcnt(n) with expcnt/lgkmcnt left alone (gfx9 encoding: vmcnt
// bits 3:0 and 15:14), as the builtin so that the compiler's own wait
// insertion knows which loads have completed
constexpr int vmcnt_imm(int n) { return ((n >> 4) << 14) | 0x0F70 | (n & 15); }
template <int N>
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt(vmcnt_imm(N)); }
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

}  // namespace qnf4
