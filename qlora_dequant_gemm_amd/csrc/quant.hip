// Quantize, double-quantize and dequantize kernels for gfx950.
//
//  k_quantize  -- one workgroup per group of 256 blocks: block absmax with a
//                 16-lane DPP reduction, nearest-level code (cell lookup with
//                 an exact fallback near thresholds), nibble packing, and
//                 optionally the double quantization of the group's
//                 constants. ("A 65B fine-tune on the GPU you already have",
//                 figures 3 and 4.)
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
// Nearest-code selection.
//
// Exact rule: v = fp32(w / absmax) (IEEE division), code = #{j : v > T_j}.
// Fast path: v' = w * rcp(absmax) is within 2.4e-7 of v. The line is cut
// into 129 cells, cell(v) = floor(64 v + 64.5); cell edges are at least
// 1.2e-3 away from every threshold (checked when the codebook is derived),
// so each cell holds at most one threshold and
//     code(v') = base[cell] + (v' > thr[cell])
// with base[cell] the thresholds in lower cells. code(v') == code(v) unless a
// threshold lies between v and v', which puts v' within 1e-6 of thr[cell];
// those (rare) elements take the exact rule.
// ---------------------------------------------------------------------------
constexpr int kCells = 129;
constexpr int64_t kQuantGrid = 512;            // k_quantize workgroups (2 per CU)

struct CellEntry {
  float thr;      // the threshold inside this cell, or +inf
  int base;       // thresholds in lower cells
};

// v in [-1 - 1e-6, 1 + 1e-6] maps to [0.49, 128.51], so truncation is the
// floor and the index is always a valid cell.
__device__ __forceinline__ int cell_of(float v) { return static_cast<int>(fmaf(v, 64.0f, 64.5f)); }

__device__ __forceinline__ uint32_t search_code(float v, const Codebook& cb) {
  // number of thresholds strictly below v, by binary search over T[0..14]
  uint32_t c = (v > cb.T[7]) ? 8u : 0u;
  float t = (c & 8u) ? cb.T[11] : cb.T[3];
  c += (v > t) ? 4u : 0u;
  const float t2a = (c & 4u) ? cb.T[13] : cb.T[9];
  const float t2b = (c & 4u) ? cb.T[5] : cb.T[1];
  t = (c & 8u) ? t2a : t2b;
  c += (v > t) ? 2u : 0u;
  const float e0 = (c & 2u) ? cb.T[2] : cb.T[0];
  const float e1 = (c & 2u) ? cb.T[6] : cb.T[4];
  const float e2 = (c & 2u) ? cb.T[10] : cb.T[8];
  const float e3 = (c & 2u) ? cb.T[14] : cb.T[12];
  const float f0 = (c & 4u) ? e1 : e0;
  const float f1 = (c & 4u) ? e3 : e2;
  t = (c & 8u) ? f1 : f0;
  c += (v > t) ? 1u : 0u;
  return c;
}

__device__ __forceinline__ uint32_t exact_code(float w, float a, const Codebook& cb) {
  const float v = (a == 0.0f) ? 0.0f : w / a;      // IEEE division
  return search_code(v, cb);
}

__device__ void build_lut(CellEntry* lut, const Codebook& cb) {
  for (int i = threadIdx.x; i < kCells; i += blockDim.x) {
    int base = 0;
    float thr = __builtin_inff();
#pragma unroll
    for (int j = 0; j < 15; ++j) {
      const int cj = cell_of(cb.T[j]);
      base += cj < i ? 1 : 0;
      if (cj == i) thr = cb.T[j];
    }
    lut[i] = CellEntry{thr, base};
  }
}

// max over the 16 lanes of a row (DPP row rotations, then quad permutes) of
// non-negative floats, compared as their bit patterns (same order)
// (every lane of these patterns has a source, so bound_ctrl never applies; it
// and the zero `old` let the compiler fold each move into the max as a DPP
// operand)
__device__ __forceinline__ float row16_max_nonneg(float a) {
  uint32_t x = __builtin_bit_cast(uint32_t, a);
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x128, 0xF, 0xF, true)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x124, 0xF, 0xF, true)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0xB1, 0xF, 0xF, true)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x4E, 0xF, 0xF, true)));
  return __builtin_bit_cast(float, x);
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

// ---------------------------------------------------------------------------
// k_quantize: a group of 256 blocks (16384 weights) at a time per 256-thread
// workgroup, groups taken grid-stride. A group is two halves of 8 rounds; a
// round is 16 blocks, 16 lanes per block and 4 consecutive weights per lane.
// The loads of the next half are in flight while the current half is coded,
// so the coding arithmetic overlaps the weight stream instead of following
// it. With DQ the group's constants are double-quantized in the same pass.
// ---------------------------------------------------------------------------
template <typename Tin, bool DQ>
__global__ __launch_bounds__(256) void k_quantize(const Tin* __restrict__ w, int64_t nblocks,
                                                  uint16_t* __restrict__ packed16,
                                                  float* __restrict__ absmax, int8_t* __restrict__ qscale,
                                                  float* __restrict__ step, Codebook cb, int64_t gstride) {
  // gstride == gridDim.x, passed as an argument: reading gridDim.x inside the
  // loop is a vector load from the dispatch packet, and waiting for it would
  // drain the prefetched weight loads
  __shared__ CellEntry lut[kCells];
  __shared__ float amax_s[256];
  __shared__ float wmax[4];
  const int t = threadIdx.x, lane16 = t & 15, sub = t >> 4;
  const int64_t ngroups = (nblocks + 255) / 256;
  int64_t g = blockIdx.x;
  if (g >= ngroups) return;
  auto nb_in = [&](int64_t gg) { return static_cast<int>(nblocks - gg * 256 < 256 ? nblocks - gg * 256 : 256); };
  // rounds 8 hh .. 8 hh + 7 of group gg
  auto load_half = [&](int64_t gg, int hh, f32x4 (&v)[8]) {
    const int nbh = nb_in(gg);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int bl = (8 * hh + i) * 16 + sub;
      const int64_t b = gg * 256 + (bl < nbh ? bl : 0);
      v[i] = Load4<Tin>::at(w + b * 64 + lane16 * 4);
    }
  };
  // fast path for the 32 elements of this thread in a half; a round with any
  // element near a threshold (or a zero / tiny block) is flagged for the exact
  // rule
  auto code_half = [&](int64_t gg, int hh, const f32x4 (&v)[8], uint32_t& redo) {
    const int nbh = nb_in(gg);
    const bool full = nbh == 256;                // every group but possibly the last
    uint16_t* pk = packed16 + (gg * 256 + sub) * 16 + lane16;   // round rd: + rd * 256
    float* am = absmax + gg * 256 + sub;                         // round rd: + rd * 16
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rd = 8 * hh + i;
      const int bl = rd * 16 + sub;
      const float a = row16_max_nonneg(fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)),
                                             fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
      const bool fast = a >= 1e-30f;             // uniform over the block's 16 lanes
      const float ra = fast ? __builtin_amdgcn_rcpf(a) : 0.0f;
      uint32_t word = 0;
      float dmin = fast ? __builtin_inff() : 0.0f;   // distance of the nearest element to its threshold
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float we = e == 0 ? v[i].x : e == 1 ? v[i].y : e == 2 ? v[i].z : v[i].w;
        const float vp = we * ra;
        const CellEntry ce = lut[cell_of(vp)];
        word |= (static_cast<uint32_t>(ce.base) + (vp > ce.thr ? 1u : 0u)) << (4 * e);
        dmin = fminf(dmin, fabsf(vp - ce.thr));   // inf - inf cannot occur: vp is finite
      }
      redo |= (dmin > 1e-6f) ? 0u : (1u << rd);
      asm volatile("" ::"v"(redo));              // keep the check in this round (register pressure)
      if (full || bl < nbh) {
        pk[rd * 256] = static_cast<uint16_t>(word);
        if (lane16 == 0) {
          am[rd * 16] = a;
          amax_s[bl] = a;
        }
      }
    }
  };
  f32x4 va[8], vb[8];
  load_half(g, 0, va);
  build_lut(lut, cb);
  __syncthreads();
  for (; g < ngroups; g += gstride) {
    const int nb_here = nb_in(g);
    load_half(g, 1, vb);
    uint32_t redo = 0;
    code_half(g, 0, va, redo);
    // next group's first half; the last group instead re-loads its own second
    // half, which is still in L2 (no branch, so no wait for this group's
    // second half before these loads issue)
    const bool more = g + gstride < ngroups;
    load_half(more ? g + gstride : g, more ? 0 : 1, va);
    code_half(g, 1, vb, redo);
    __syncthreads();                             // amax_s complete
    if (redo) {                                  // rare: exact rule for the flagged rounds
#pragma unroll 1
      for (int rd = 0; rd < 16; ++rd) {
        const int bl = rd * 16 + sub;
        if (!(redo & (1u << rd)) || bl >= nb_here) continue;
        const int64_t b = g * 256 + bl;
        const f32x4 x = Load4<Tin>::at(w + b * 64 + lane16 * 4);
        const float a = amax_s[bl];
        uint32_t word = 0;
#pragma unroll 1
        for (int e = 0; e < 4; ++e) {
          const float we = e == 0 ? x.x : e == 1 ? x.y : e == 2 ? x.z : x.w;
          word |= exact_code(we, a, cb) << (4 * e);
        }
        packed16[b * 16 + lane16] = static_cast<uint16_t>(word);
      }
    }
    if (DQ) {
      // double quantization of this group's constants (same arithmetic as k_dq_scales)
      const float a = t < nb_here ? amax_s[t] : 0.0f;
      float m = a;
      for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
      if ((t & 63) == 0) wmax[t >> 6] = m;
      __syncthreads();
      m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
      const float d = m / 127.0f;
      if (t < nb_here) {
        int q = 0;
        if (d != 0.0f) {
          const float r = fminf(fmaxf(__builtin_rintf(a / d), -127.0f), 127.0f);
          q = static_cast<int>(r);
        }
        qscale[g * 256 + t] = static_cast<int8_t>(q);
      }
      if (t == 0) step[g] = d;
    }
    __syncthreads();                             // amax_s / wmax free for the next group
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
// DQ == false: the block constants are the fp32 absmax values themselves
// (storage without double quantization).
template <bool DQ>
__global__ __launch_bounds__(256) void k_dequant(const u32x4* __restrict__ packed, const int8_t* __restrict__ qscale,
                                                 const float* __restrict__ step, const float* __restrict__ absmax,
                                                 int64_t nchunks, u32x4* __restrict__ out, Codebook cb) {
  const int64_t first = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t c = first; c < nchunks; c += stride) {
    const u32x4 p = packed[c];
    const int64_t blk = c >> 1;                // 2 chunks of 32 codes per block
    const float s = DQ ? block_scale(qscale[blk], step[blk >> 8]) : absmax[blk];
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
                           int8_t* qscale, float* step, const Codebook& cb, hipStream_t stream) {
  const int64_t nb = numel / 64;
  // two groups or more per workgroup once there are enough groups to fill
  // the chip: each workgroup then overlaps one group's coding with the next
  // group's loads
  const int64_t ngroups = (nb + 255) / 256;
  const dim3 grid(static_cast<unsigned>(ngroups < kQuantGrid ? ngroups : kQuantGrid));
  uint16_t* p16 = reinterpret_cast<uint16_t*>(packed);
  const bool dq = qscale != nullptr;
  if (wdt == 0) {
    const float* wf = static_cast<const float*>(w);
    if (dq)
      hipLaunchKernelGGL((k_quantize<float, true>), grid, dim3(256), 0, stream, wf, nb, p16, absmax, qscale, step, cb,
                         static_cast<int64_t>(grid.x));
    else
      hipLaunchKernelGGL((k_quantize<float, false>), grid, dim3(256), 0, stream, wf, nb, p16, absmax, qscale, step, cb,
                         static_cast<int64_t>(grid.x));
  } else {
    const uint16_t* wb = static_cast<const uint16_t*>(w);
    if (dq)
      hipLaunchKernelGGL((k_quantize<uint16_t, true>), grid, dim3(256), 0, stream, wb, nb, p16, absmax, qscale, step, cb,
                         static_cast<int64_t>(grid.x));
    else
      hipLaunchKernelGGL((k_quantize<uint16_t, false>), grid, dim3(256), 0, stream, wb, nb, p16, absmax, qscale, step, cb,
                         static_cast<int64_t>(grid.x));
  }
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
                          uint16_t* out, const Codebook& cb, hipStream_t stream, const float* absmax) {
  const int64_t nchunks = numel / 32;
  const int grid = grid_for(nchunks, 256);
  if (qscale)
    hipLaunchKernelGGL(k_dequant<true>, dim3(grid), dim3(256), 0, stream, reinterpret_cast<const u32x4*>(packed),
                       qscale, step, nullptr, nchunks, reinterpret_cast<u32x4*>(out), cb);
  else
    hipLaunchKernelGGL(k_dequant<false>, dim3(grid), dim3(256), 0, stream, reinterpret_cast<const u32x4*>(packed),
                       nullptr, nullptr, absmax, nchunks, reinterpret_cast<u32x4*>(out), cb);
  return hipGetLastError();
}

}  // namespace qnf4
