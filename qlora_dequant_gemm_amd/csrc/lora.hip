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

// ---------------------------------------------------------------------------
// Large M (and the transposed outputs of the adapter gradients): 64-row tiles
// x KS splits of the contraction. Wave w owns rows 16w .. 16w + 15 of the
// tile and every rank tile, so each adapter fragment is used by 64 rows of
// the workgroup (once per wave, from L1/L2); all loads of a group of GS steps
// are issued before its MFMAs. Operands come through buffer descriptors: rows
// past M read as zero, and so do adapter rows past r; a step's lanes past Kc
// (Kc % 32 != 0) get a zeroed adapter fragment. KS == 1 writes bf16 directly
// (padding ranks up to rp zero), else fp32 partials [KS][Mr][16 NT] that
// k_down_finish sums in order.
// ---------------------------------------------------------------------------
constexpr int kBufWord3 = 0x00020000;          // raw buffer descriptor word 3 on gfx9-family parts

template <int NT, int GS>
__global__ __launch_bounds__(256) void k_down(const uint16_t* in, int64_t M, int64_t Kc, const uint16_t* W, int r,
                                              int rp, int64_t sps, int KS, float* __restrict__ part,
                                              uint16_t* __restrict__ out, int64_t ldt) {
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int tile = blockIdx.x / KS, ks = blockIdx.x % KS;
  const int64_t m0 = static_cast<int64_t>(tile) * 64;
  const int64_t nsteps = cdiv(Kc, 32);
  const int64_t st0 = ks * sps, st1 = imin(nsteps, st0 + sps);
  const int64_t rows_valid = imin(64, M - m0);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(in + m0 * Kc), 0, static_cast<int>(rows_valid * Kc * 2), kBufWord3);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(W), 0, static_cast<int>(static_cast<int64_t>(r) * Kc * 2), kBufWord3);
  const uint32_t xoff = static_cast<uint32_t>(((16 * w + c) * Kc + 8 * g) * 2);
  uint32_t woff[NT];
#pragma unroll
  for (int jt = 0; jt < NT; ++jt) woff[jt] = static_cast<uint32_t>(((16 * jt + c) * Kc + 8 * g) * 2);
  f32x4 acc[NT];
#pragma unroll
  for (int jt = 0; jt < NT; ++jt) acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int64_t st = st0; st < st1; st += GS) {
    u32x4 xa[GS], wa[GS][NT];
#pragma unroll
    for (int u = 0; u < GS; ++u) {
      const uint32_t so = static_cast<uint32_t>(imin(st + u, st1 - 1) * 64);
      xa[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, xoff, so, 0));
#pragma unroll
      for (int jt = 0; jt < NT; ++jt)
        wa[u][jt] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, woff[jt], so, 0));
    }
#pragma unroll
    for (int u = 0; u < GS; ++u) {
      // a clamped repeat of the last step, or lanes past Kc: no contribution
      const bool live = st + u < st1 && (st + u) * 32 + 8 * g < Kc;
#pragma unroll
      for (int jt = 0; jt < NT; ++jt) {
        const u32x4 b = live ? wa[u][jt] : u32x4{0u, 0u, 0u, 0u};
        acc[jt] = mfma16(as_bf16x8(xa[u]), as_bf16x8(b), acc[jt]);
      }
    }
  }
  // lane holds rows 16w + 4g + v of the tile, rank 16 jt + c
  if (KS > 1) {
    float* dst = part + (static_cast<int64_t>(ks) * (cdiv(M, 64) * 64) + m0 + 16 * w + 4 * g) * (16 * NT);
#pragma unroll
    for (int jt = 0; jt < NT; ++jt)
#pragma unroll
      for (int v = 0; v < 4; ++v) dst[v * 16 * NT + 16 * jt + c] = acc[jt][v];
    return;
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t m = m0 + 16 * w + 4 * g + v;
    if (ldt) {
      if (m >= ldt) continue;
#pragma unroll
      for (int jt = 0; jt < NT; ++jt)
        if (16 * jt + c < rp) out[(16 * jt + c) * ldt + m] = m < M ? bf16_bits(acc[jt][v]) : uint16_t{0};
      for (int j = 16 * NT + c; j < rp; j += 16) out[j * ldt + m] = 0;
    } else if (m < M) {
#pragma unroll
      for (int jt = 0; jt < NT; ++jt)
        if (16 * jt + c < rp) out[m * rp + 16 * jt + c] = bf16_bits(acc[jt][v]);
      for (int j = 16 * NT + c; j < rp; j += 16) out[m * rp + j] = 0;
    }
  }
}

// ---------------------------------------------------------------------------
// Row-streaming form for the matmul paths (M > 16, output [M][rp]): one
// workgroup per 16 rows of `in`, its eight waves taking interleaved 64-deep
// chunks of the contraction (wave w: chunks w, w + 8, ...), so the workgroup
// streams its rows front to back with 8 GS chunks of each row in flight and
// no split partials leave the chip; the eight waves' 16 x 16 RT accumulators
// are summed through LDS in wave order.
// 16x16x32 bf16 MFMA: in a 64-deep chunk, lane (g, c) supplies row c's
// elements [16 g, 16 g + 16) as the k-slots of two MFMAs, and the adapter
// row 16 jt + c the same elements (a contraction is order-free). Kc % 8 == 0:
// 8-element pieces past Kc are zeroed; rows past M and adapter rows past r
// read as zero through the descriptors.
// ---------------------------------------------------------------------------
constexpr int kDownWaves = 8;

template <int RT, int GS>
__global__ __launch_bounds__(64 * kDownWaves) void k_down_rows(const uint16_t* in, int M, int Kc, const uint16_t* W, int r,
                                                   int rp, uint16_t* __restrict__ out, int ldt) {
  __shared__ f32x4 red[kDownWaves][RT][64];
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int m0 = blockIdx.x * 16;
  const int rows_valid = M - m0 < 0 ? 0 : (M - m0 < 16 ? M - m0 : 16);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(in + static_cast<int64_t>(m0) * Kc), 0, rows_valid * Kc * 2, kBufWord3);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(W), 0, r * Kc * 2,
                                                                      kBufWord3);
  const int nchunk = (Kc + 63) / 64;
  const uint32_t xo = static_cast<uint32_t>((c * Kc + 16 * g) * 2);
  uint32_t wo[RT];
#pragma unroll
  for (int jt = 0; jt < RT; ++jt) wo[jt] = static_cast<uint32_t>(((16 * jt + c) * Kc + 16 * g) * 2);
  f32x4 acc[RT];
#pragma unroll
  for (int jt = 0; jt < RT; ++jt) acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const u32x4 zero = {0u, 0u, 0u, 0u};
  // GS chunks per round, all their loads issued before their MFMAs
  for (int q0 = w; q0 < nchunk; q0 += kDownWaves * GS) {
    u32x4 xa[GS][2], wa[GS][RT][2];
#pragma unroll
    for (int u = 0; u < GS; ++u) {
      const int q = q0 + kDownWaves * u < nchunk ? q0 + kDownWaves * u : nchunk - 1;
      const uint32_t so = static_cast<uint32_t>(q * 128);
      xa[u][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, xo, so, 0));
      xa[u][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, xo + 16, so, 0));
#pragma unroll
      for (int jt = 0; jt < RT; ++jt) {
        wa[u][jt][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, wo[jt], so, 0));
        wa[u][jt][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, wo[jt] + 16, so, 0));
      }
    }
#pragma unroll
    for (int u = 0; u < GS; ++u) {
      const int q = q0 + kDownWaves * u;
      const int k = q * 64 + 16 * g;
      // a repeated last chunk, or pieces past Kc, contribute nothing
      const bool live0 = q < nchunk && k < Kc, live1 = q < nchunk && k + 8 < Kc;
      const u32x4 x0 = live0 ? xa[u][0] : zero, x1 = live1 ? xa[u][1] : zero;
#pragma unroll
      for (int jt = 0; jt < RT; ++jt) {
        acc[jt] = mfma16(as_bf16x8(x0), as_bf16x8(live0 ? wa[u][jt][0] : zero), acc[jt]);
        acc[jt] = mfma16(as_bf16x8(x1), as_bf16x8(live1 ? wa[u][jt][1] : zero), acc[jt]);
      }
    }
  }
#pragma unroll
  for (int jt = 0; jt < RT; ++jt) red[w][jt][lane] = acc[jt];
  __syncthreads();
  // lane (g, c) of a fragment holds rows 4 g + v, rank 16 jt + c; ldt > 0:
  // written transposed, [rp][ldt], with the rows past M (zero sums) as well
  for (int e = t; e < 16 * rp; e += 64 * kDownWaves) {
    const int row = ldt ? e & 15 : e / rp, j = ldt ? e >> 4 : e - (e / rp) * rp;
    if (ldt ? m0 + row >= ldt : row >= rows_valid) continue;
    float sum = 0.f;
    if (j < 16 * RT) {
      const int jt = j >> 4, l = ((row >> 2) << 4) | (j & 15);
      const int v = row & 3;
#pragma unroll
      for (int ww = 0; ww < kDownWaves; ++ww) sum += red[ww][jt][l][v];
    }
    if (ldt)
      out[static_cast<int64_t>(j) * ldt + m0 + row] = bf16_bits(sum);
    else
      out[static_cast<int64_t>(m0 + row) * rp + j] = bf16_bits(sum);
  }
}

// Sum of the KS split partials in order, rounded to bf16, written [M][rp] or
// transposed [rp][ldt] (rows past M and ranks past 16 nt zero).
__global__ __launch_bounds__(256) void k_down_finish(const float* __restrict__ part, int KS, int64_t M,
                                                     int64_t Mr, int cols, int rp, uint16_t* __restrict__ out,
                                                     int64_t ldt) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t rows = ldt ? ldt : M;
  if (idx >= rows * rp) return;
  const int64_t m = ldt ? idx % ldt : idx / rp;
  const int j = static_cast<int>(ldt ? idx / ldt : idx % rp);
  float sum = 0.f;
  if (m < M && j < cols)
    for (int ks = 0; ks < KS; ++ks) sum += part[(ks * Mr + m) * cols + j];
  out[ldt ? j * ldt + m : m * rp + j] = bf16_bits(sum);
}

// B [N][r] -> Bt [r][N] (the backward contracts over N, so it reads the
// adapter row-major through this copy): 64 rows of B (one contiguous run of
// 128 r bytes) staged in LDS, then each rank's 64 values written contiguously.
__global__ __launch_bounds__(256) void k_adapter_t(const uint16_t* __restrict__ B, int64_t N, int r,
                                                   uint16_t* __restrict__ Bt) {
  __shared__ uint16_t tileb[64 * 128];
  const int t = threadIdx.x;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 64;
  const int nrows = static_cast<int>(imin(64, N - n0));
  const int n16 = nrows * r / 8;                 // 16-byte pieces (N % 8 == 0: r * nrows % 8 == 0)
  const u32x4* src = reinterpret_cast<const u32x4*>(B + n0 * r);
  for (int i = t; i < n16; i += 256) reinterpret_cast<u32x4*>(tileb)[i] = src[i];
  __syncthreads();
  for (int i = t; i < r * 64; i += 256) {
    const int j = i >> 6, nn = i & 63;
    if (nn < nrows) Bt[j * N + n0 + nn] = tileb[nn * r + j];
  }
}

hipError_t launch_lora_down(bool wrow, const uint16_t* in, int64_t M, int64_t Kc, const uint16_t* W, int r,
                            void* out, hipStream_t stream, uint16_t* wt, float* part, int64_t ldt) {
  const int rp = static_cast<int>(rank_pad(r));
  const uint16_t* Wr = W;
  if (!wrow) {
    hipLaunchKernelGGL(k_adapter_t, dim3(static_cast<unsigned>(cdiv(Kc, 64))), dim3(256), 0, stream, W, Kc, r, wt);
    Wr = wt;
  }
  if (M > 16) {
    // row-streaming form, no split partials (ldt: the rows up to ldt too)
    const unsigned grid16 = static_cast<unsigned>(cdiv(ldt ? ldt : M, 16));
    const int mi = static_cast<int>(M), kci = static_cast<int>(Kc), lt = static_cast<int>(ldt);
    uint16_t* o16 = static_cast<uint16_t*>(out);
    const int nt = down_nt(r);
    if (nt == 1)
      hipLaunchKernelGGL(HIP_KERNEL_NAME(k_down_rows<1, 4>), dim3(grid16), dim3(64 * kDownWaves), 0, stream, in, mi, kci, Wr, r,
                         rp, o16, lt);
    else if (nt == 2)
      hipLaunchKernelGGL(HIP_KERNEL_NAME(k_down_rows<2, 4>), dim3(grid16), dim3(64 * kDownWaves), 0, stream, in, mi, kci, Wr, r,
                         rp, o16, lt);
    else if (nt == 4)
      hipLaunchKernelGGL(HIP_KERNEL_NAME(k_down_rows<4, 2>), dim3(grid16), dim3(64 * kDownWaves), 0, stream, in, mi, kci, Wr, r,
                         rp, o16, lt);
    else
      hipLaunchKernelGGL(HIP_KERNEL_NAME(k_down_rows<8, 1>), dim3(grid16), dim3(64 * kDownWaves), 0, stream, in, mi, kci, Wr, r,
                         rp, o16, lt);
    return hipGetLastError();
  }
  const DownPlan p = down_plan(M, Kc, r);
  const unsigned grid = static_cast<unsigned>(cdiv(M, 64) * p.KS);
  const int KS = static_cast<int>(p.KS);
  uint16_t* o = static_cast<uint16_t*>(out);
#define QNF4_DOWN(NTV, GSV)                                                                                      \
  hipLaunchKernelGGL(HIP_KERNEL_NAME(k_down<NTV, GSV>), dim3(grid), dim3(256), 0, stream, in, M, Kc, Wr, r, rp, \
                     p.sps, KS, part, o, ldt)
  if (p.nt == 1)
    QNF4_DOWN(1, 8);
  else if (p.nt == 2)
    QNF4_DOWN(2, 8);
  else if (p.nt == 4)
    QNF4_DOWN(4, 4);
  else
    QNF4_DOWN(8, 2);
#undef QNF4_DOWN
  if (KS > 1) {
    const int64_t n = (ldt ? ldt : M) * rp;
    hipLaunchKernelGGL(k_down_finish, dim3(static_cast<unsigned>(cdiv(n, 256))), dim3(256), 0, stream, part, KS, M,
                       p.Mr, 16 * p.nt, rp, o, ldt);
  }
  return hipGetLastError();
}

}  // namespace qnf4
