// Quantize, double-quantize and dequantize kernels for gfx950.
//
//  k_quantize  -- block absmax with a 16-lane reduction, fp32 normalisation,
//                 nearest-level code by binary search on the thresholds,
//                 nibble packing. ("A 65B fine-tune on the GPU you already
//                 have", figures 3 and 4.)
//  k_dq_scales -- one workgroup per group of 256 block constants: group max,
//                 step = max / 127, int8 codes. (same page, figure 4.)
//  k_dequant   -- packed codes + int8 scales + fp32 steps -> bf16, with the
//                 same per-block table decode the fused GEMMs use.
//                 (same page, figure 2.)
// All three are HBM-bound streaming kernels: vector loads of 16 bytes per
// lane, grid-stride loops, and no shared-memory traffic beyond one reduction.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"
#include "kernels.hpp"

namespace qnf4 {

// ---------------------------------------------------------------------------
// k_quantize: 16 lanes per 64-weight block, 4 consecutive weights per lane.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t nearest_code(float v, const Codebook& cb) {
  // number of thresholds strictly below v, by binary search over T[0..14]
  uint32_t c = (v > cb.T[7]) ? 8u : 0u;
  float t = (c & 8u) ? cb.T[11] : cb.T[3];
  c += (v > t) ? 4u : 0u;
  float t2a = (c & 4u) ? cb.T[13] : cb.T[9];
  float t2b = (c & 4u) ? cb.T[5] : cb.T[1];
  t = (c & 8u) ? t2a : t2b;
  c += (v > t) ? 2u : 0u;
  // c in {0,2,...,14}: compare with T[c]
  float e0 = (c & 2u) ? cb.T[2] : cb.T[0];
  float e1 = (c & 2u) ? cb.T[6] : cb.T[4];
  float e2 = (c & 2u) ? cb.T[10] : cb.T[8];
  float e3 = (c & 2u) ? cb.T[14] : cb.T[12];
  float f0 = (c & 4u) ? e1 : e0;
  float f1 = (c & 4u) ? e3 : e2;
  t = (c & 8u) ? f1 : f0;
  c += (v > t) ? 1u : 0u;
  return c;
}

template <typename Tin>
struct Load4;
template <>
struct Load4<float> {
  __device__ static f32x4 at(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
};
template <>
struct Load4<uint16_t> {
  __device__ static f32x4 at(const uint16_t* p) {
    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
    f32x4 r;
    r.x = bf16_lo(v.x);
    r.y = bf16_hi(v.x);
    r.z = bf16_lo(v.y);
    r.w = bf16_hi(v.y);
    return r;
  }
};

template <typename Tin>
__global__ __launch_bounds__(256) void k_quantize(const Tin* __restrict__ w, int64_t nblocks,
                                                  uint16_t* __restrict__ packed16,
                                                  float* __restrict__ absmax, Codebook cb) {
  const int lane16 = threadIdx.x & 15;
  const int64_t first = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) >> 4;
  const int64_t stride = (static_cast<int64_t>(gridDim.x) * blockDim.x) >> 4;
  for (int64_t b = first; b < nblocks; b += stride) {
    const f32x4 v = Load4<Tin>::at(w + b * 64 + lane16 * 4);
    float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    // max over the 16 lanes of this block (xor offsets stay inside the group)
    a = fmaxf(a, __shfl_xor(a, 8, 16));
    a = fmaxf(a, __shfl_xor(a, 4, 16));
    a = fmaxf(a, __shfl_xor(a, 2, 16));
    a = fmaxf(a, __shfl_xor(a, 1, 16));
    uint32_t c0, c1, c2, c3;
    if (a == 0.0f) {
      c0 = c1 = c2 = c3 = nearest_code(0.0f, cb);
    } else {
      c0 = nearest_code(v.x / a, cb);          // IEEE division (correctly rounded)
      c1 = nearest_code(v.y / a, cb);
      c2 = nearest_code(v.z / a, cb);
      c3 = nearest_code(v.w / a, cb);
    }
    const uint32_t word = c0 | (c1 << 4) | (c2 << 8) | (c3 << 12);
    packed16[b * 16 + lane16] = static_cast<uint16_t>(word);   // 32 bytes per block
    if (lane16 == 0) absmax[b] = a;
  }
}

// ---------------------------------------------------------------------------
// k_dq_scales: one 256-thread workgroup per group of 256 block constants.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_dq_scales(const float* __restrict__ absmax, int64_t nblocks,
                                                   int8_t* __restrict__ qscale,
                                                   float* __restrict__ step) {
  __shared__ float wmax[4];
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const float a = (i < nblocks) ? absmax[i] : 0.0f;
  float m = a;
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float d = m / 127.0f;                  // IEEE division
  if (i < nblocks) {
    int q = 0;
    if (d != 0.0f) {
      float r = __builtin_rintf(a / d);        // round half to even
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      q = static_cast<int>(r);
    }
    qscale[i] = static_cast<int8_t>(q);
  }
  if (threadIdx.x == 0) step[blockIdx.x] = d;
}

// ---------------------------------------------------------------------------
// k_dequant: each lane turns 16 packed bytes (32 codes, half a block) into
// 32 bf16 (64 bytes).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_dequant(const u32x4* __restrict__ packed, const int8_t* __restrict__ qscale,
                                                 const float* __restrict__ step, int64_t nchunks,
                                                 u32x4* __restrict__ out, Codebook cb) {
  const int64_t first = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t c = first; c < nchunks; c += stride) {
    const u32x4 p = packed[c];
    const int64_t blk = c >> 1;                // 2 chunks of 32 codes per block
    const float s = block_scale(qscale[blk], step[blk >> 8]);
    const MagTable t = make_table(cb, s);
    out[c * 4 + 0] = decode8(p.x, t);
    out[c * 4 + 1] = decode8(p.y, t);
    out[c * 4 + 2] = decode8(p.z, t);
    out[c * 4 + 3] = decode8(p.w, t);
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static int grid_for(int64_t work_items, int per_block) {
  int64_t g = (work_items + per_block - 1) / per_block;
  const int64_t cap = 256 * 32;                // 32 workgroups per CU at most
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return static_cast<int>(g);
}

hipError_t launch_quantize(const void* w, int wdt, int64_t numel, uint8_t* packed, float* absmax,
                           const Codebook& cb, hipStream_t stream) {
  const int64_t nb = numel / 64;
  const int grid = grid_for(nb, 16);           // 16 blocks per 256-thread workgroup
  if (wdt == 0)
    hipLaunchKernelGGL(k_quantize<float>, dim3(grid), dim3(256), 0, stream,
                       static_cast<const float*>(w), nb, reinterpret_cast<uint16_t*>(packed), absmax, cb);
  else
    hipLaunchKernelGGL(k_quantize<uint16_t>, dim3(grid), dim3(256), 0, stream,
                       static_cast<const uint16_t*>(w), nb, reinterpret_cast<uint16_t*>(packed), absmax, cb);
  return hipGetLastError();
}

hipError_t launch_dq_scales(const float* absmax, int64_t nblocks, int8_t* qscale, float* step,
                            hipStream_t stream) {
  const int64_t ng = (nblocks + 255) / 256;
  hipLaunchKernelGGL(k_dq_scales, dim3(static_cast<unsigned>(ng)), dim3(256), 0, stream, absmax, nblocks,
                     qscale, step);
  return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* packed, const int8_t* qscale, const float* step, int64_t numel,
                          uint16_t* out, const Codebook& cb, hipStream_t stream) {
  const int64_t nchunks = numel / 32;
  const int grid = grid_for(nchunks, 256);
  hipLaunchKernelGGL(k_dequant, dim3(grid), dim3(256), 0, stream, reinterpret_cast<const u32x4*>(packed),
                     qscale, step, nchunks, reinterpret_cast<u32x4*>(out), cb);
  return hipGetLastError();
}

}  // namespace qnf4
