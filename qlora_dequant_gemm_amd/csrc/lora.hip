// Rank-r LoRA down-projections for gfx950: t = x . A^T (forward, contraction
// over K) and u = dY . B (backward, contraction over N), on 16x16x32 bf16
// MFMA with fp32 accumulation. The LoRA update itself is the standard one for
// the r / lora_alpha knobs ("QLoRA and Quantized Training", "In code"; "A 65B
// fine-tune on the GPU you already have", figure 2: same low-rank update).
//
// The adapter matrix W(j, k) is either row-major over the contraction
// (WROW: A [r][K]) or column-major (B [N][r], read as W(j, n) = B[n][j]).
// Columns j >= r are zero, so the output is padded to rp = roundup(r, 32).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mm_common.hpp"

namespace qnf4 {

// 8 consecutive contraction values W(j, k..k+7) of adapter column j.
template <bool WROW>
__device__ __forceinline__ u32x4 adapter8(const uint16_t* __restrict__ W, int64_t Kc, int r, int j, int64_t k) {
  if (j >= r || k >= Kc) return u32x4{0u, 0u, 0u, 0u};
  if (WROW) return ld16(W + static_cast<int64_t>(j) * Kc + k);   // Kc % 8 == 0, rows 16-byte aligned
  uint32_t v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t lo = W[(k + 2 * e) * r + j];
    const uint32_t hi = W[(k + 2 * e + 1) * r + j];
    v[e] = lo | (hi << 16);
  }
  return u32x4{v[0], v[1], v[2], v[3]};
}

// ---------------------------------------------------------------------------
// Large M: out bf16 [M][rp]. Grid ceil(M/16): the 4 waves of a workgroup share
// 16 rows and take the 32-deep contraction steps round robin (operands straight
// from global memory; the adapter stays in L2), then reduce through LDS.
// ---------------------------------------------------------------------------
// NT: 16-wide rank tiles holding real ranks (ceil(r / 16)); the padding
// columns up to rp are written as zero. TRANS writes the result transposed,
// out [rp][ldt] with ldt >= M, rows m in [M, ldt) zero (the grid then covers
// ldt / 16 row tiles). Each wave takes 32-deep contraction
// steps round robin in groups of 8, all of a group's loads issued before its
// MFMAs, so that enough loads are in flight to stream `in` from HBM.
template <int NT, bool TRANS>
__global__ __launch_bounds__(256) void k_lora_down(const uint16_t* __restrict__ in, int64_t M, int64_t Kc,
                                                   const uint16_t* __restrict__ W, int r, int rp,
                                                   uint16_t* __restrict__ out, int64_t ldt) {
  __shared__ f32x4 red[4][8][64];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int ntile = rp / 16;
  const uint16_t* in_row = in + imin(m0 + c, M - 1) * Kc;
  const int64_t nsteps = cdiv(Kc, 32);
  f32x4 acc[8];
#pragma unroll
  for (int jt = 0; jt < 8; ++jt) acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int kGroup = 8;
  for (int64_t st0 = w * kGroup; st0 < nsteps; st0 += 4 * kGroup) {
    u32x4 xa[kGroup], wa[kGroup][NT];
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      const int64_t k = (st0 + u) * 32 + 8 * g;
      const bool kin = st0 + u < nsteps && k < Kc;
      xa[u] = kin ? ld16(in_row + k) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int jt = 0; jt < NT; ++jt) wa[u][jt] = kin ? adapter8<true>(W, Kc, r, 16 * jt + c, k) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kGroup; ++u)
#pragma unroll
      for (int jt = 0; jt < NT; ++jt) acc[jt] = mfma16(as_bf16x8(xa[u]), as_bf16x8(wa[u][jt]), acc[jt]);
  }
#pragma unroll
  for (int jt = 0; jt < 8; ++jt)
    if (jt < ntile) red[w][jt][lane] = acc[jt];
  __syncthreads();
  for (int idx = t; idx < ntile * 64; idx += 256) {
    const int jt = idx >> 6, ln = idx & 63;
    const f32x4 sum = red[0][jt][ln] + red[1][jt][ln] + red[2][jt][ln] + red[3][jt][ln];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t m = m0 + 4 * (ln >> 4) + v;
      if (TRANS) {
        if (m < ldt) out[(16 * jt + (ln & 15)) * ldt + m] = m < M ? bf16_bits(sum[v]) : uint16_t{0};
      } else if (m < M) {
        out[m * rp + 16 * jt + (ln & 15)] = bf16_bits(sum[v]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Small M (<= 16): fp32 partial sums [S][M][rp]. Grid S workgroups of 8 waves;
// workgroup s owns a contiguous range of 32-deep steps and its waves take
// them round robin, so every load of the workgroup is issued up front.
// ---------------------------------------------------------------------------
template <bool WROW>
__global__ __launch_bounds__(512) void k_lora_down_small(const uint16_t* __restrict__ in, int64_t M, int64_t Kc,
                                                         const uint16_t* __restrict__ W, int r, int rp, int S,
                                                         float* __restrict__ out) {
  __shared__ f32x4 red[8][8][64];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int s = blockIdx.x;
  const int ntile = rp / 16;
  const int64_t nsteps = cdiv(Kc, 32);
  const int64_t beg = s * nsteps / S, end = (s + 1) * nsteps / S;
  const uint16_t* in_row = in + imin(static_cast<int64_t>(c), M - 1) * Kc;
  f32x4 acc[8];
#pragma unroll
  for (int jt = 0; jt < 8; ++jt) acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
  for (int64_t st = beg + w; st < end; st += 8) {
    const int64_t k = st * 32 + 8 * g;
    const bf16x8 a = as_bf16x8(k < Kc ? ld16(in_row + k) : u32x4{0u, 0u, 0u, 0u});
#pragma unroll
    for (int jt = 0; jt < 8; ++jt)
      if (jt < ntile) acc[jt] = mfma16(a, as_bf16x8(adapter8<WROW>(W, Kc, r, 16 * jt + c, k)), acc[jt]);
  }
#pragma unroll
  for (int jt = 0; jt < 8; ++jt)
    if (jt < ntile) red[w][jt][lane] = acc[jt];
  __syncthreads();
  for (int idx = t; idx < ntile * 64; idx += 512) {
    const int jt = idx >> 6, ln = idx & 63;
    f32x4 sum = red[0][jt][ln];
#pragma unroll
    for (int i = 1; i < 8; ++i) sum += red[i][jt][ln];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t m = 4 * (ln >> 4) + v;
      if (m < M) out[(s * M + m) * rp + 16 * jt + (ln & 15)] = sum[v];
    }
  }
}

// B [N][r] -> Bt [r][N] (the large-M backward contracts over N, so it reads
// the adapter row-major through this copy)
__global__ __launch_bounds__(256) void k_adapter_t(const uint16_t* __restrict__ B, int64_t N, int r,
                                                   uint16_t* __restrict__ Bt) {
  const int64_t n = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (n >= N) return;
  for (int j = 0; j < r; ++j) Bt[static_cast<int64_t>(j) * N + n] = B[n * r + j];
}

hipError_t launch_lora_down(bool wrow, const uint16_t* in, int64_t M, int64_t Kc, const uint16_t* W, int r,
                            void* out, hipStream_t stream, uint16_t* wt, int64_t ldt) {
  const int rp = static_cast<int>(rank_pad(r));
  if (M <= kSmallM && ldt == 0) {
    const int S = static_cast<int>(lora_splits(M, Kc));
    if (wrow)
      hipLaunchKernelGGL(k_lora_down_small<true>, dim3(S), dim3(512), 0, stream, in, M, Kc, W, r, rp, S,
                         static_cast<float*>(out));
    else
      hipLaunchKernelGGL(k_lora_down_small<false>, dim3(S), dim3(512), 0, stream, in, M, Kc, W, r, rp, S,
                         static_cast<float*>(out));
  } else {
    const unsigned grid = static_cast<unsigned>(cdiv(ldt ? ldt : M, 16));
    const uint16_t* Wr = W;
    if (!wrow) {
      hipLaunchKernelGGL(k_adapter_t, dim3(static_cast<unsigned>(cdiv(Kc, 256))), dim3(256), 0, stream, W, Kc, r,
                         wt);
      Wr = wt;
    }
    const int nt = (r + 15) / 16;
#define QNF4_LDOWN(NTV)                                                                                     \
  if (ldt)                                                                                                  \
    hipLaunchKernelGGL(HIP_KERNEL_NAME(k_lora_down<NTV, true>), dim3(grid), dim3(256), 0, stream, in, M, Kc, \
                       Wr, r, rp, static_cast<uint16_t*>(out), ldt);                                        \
  else                                                                                                      \
    hipLaunchKernelGGL(HIP_KERNEL_NAME(k_lora_down<NTV, false>), dim3(grid), dim3(256), 0, stream, in, M, Kc, \
                       Wr, r, rp, static_cast<uint16_t*>(out), ldt)
    if (nt <= 1)
      QNF4_LDOWN(1);
    else if (nt == 2)
      QNF4_LDOWN(2);
    else if (nt <= 4)
      QNF4_LDOWN(4);
    else
      QNF4_LDOWN(8);
#undef QNF4_LDOWN
  }
  return hipGetLastError();
}

}  // namespace qnf4
