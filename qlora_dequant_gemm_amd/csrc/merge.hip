// Merge of the LoRA adapter into one dense bf16 weight for deployment: the
// update is the usual low-rank one, so it folds back into the weights ("QLoRA"
// (techbytebybyte), "Curiosity question: is the final model permanently
// 4-bit?" and "Training setup versus deployment setup"; "A 65B fine-tune on
// the GPU you already have", figure 2):
//     out[n][k] = bf16( W'[n][k] + (alpha / r) . sum_j B[n][j] . A[j][k] )
// with W' the dequantized bf16 weight (the exact arithmetic of
// qlora_nf4_dequant). The rank-r sum is taken in fp32 with fused multiply-adds
// in j order, then one fused multiply-add with the scale onto W' and one
// rounding to bf16.
//
// k_merge: a wave owns 4 weight rows and 512 columns (8 per lane, one packed
// code dword and one 16-byte output per row); the adapter row fragment
// A[j][k .. k+7] is loaded once per j and used for the 4 rows, whose B values
// are wave-uniform scalars.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mm_common.hpp"

namespace qnf4 {

namespace {
constexpr int kMergeRows = 4;           // weight rows per wave
constexpr int kMergeCols = 512;         // columns per wave (8 per lane)
}  // namespace

__global__ __launch_bounds__(256) void k_merge(const uint8_t* __restrict__ packed, const int8_t* __restrict__ qscale,
                                               const float* __restrict__ step, int64_t N, int64_t K,
                                               const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                               int r, float scale, uint16_t* __restrict__ out, Codebook cb,
                                               int64_t col_chunks) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t rg = wid / col_chunks, cc = wid % col_chunks;
  const int64_t n0 = rg * kMergeRows;
  const int64_t k = cc * kMergeCols + 8 * lane;
  if (n0 >= N || k >= K) return;
  float acc[kMergeRows][8];
#pragma unroll
  for (int i = 0; i < kMergeRows; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;
  for (int j = 0; j < r; ++j) {
    const u32x4 a = ld16(A + static_cast<int64_t>(j) * K + k);
    float av[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      av[2 * e] = bf16_lo(a[e]);
      av[2 * e + 1] = bf16_hi(a[e]);
    }
#pragma unroll
    for (int i = 0; i < kMergeRows; ++i) {
      const int64_t n = n0 + i < N ? n0 + i : N - 1;
      const float b = __builtin_bit_cast(float, static_cast<uint32_t>(B[n * r + j]) << 16);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[i][e] = fmaf(b, av[e], acc[i][e]);
    }
  }
#pragma unroll
  for (int i = 0; i < kMergeRows; ++i) {
    const int64_t n = n0 + i;
    if (n >= N) break;
    const int64_t e0 = n * K + k;                               // first of the lane's 8 weights
    const uint32_t codes = *reinterpret_cast<const uint32_t*>(packed + e0 / 2);
    const int64_t blk = e0 / 64;
    const MagTable t = make_table(cb, block_scale(qscale[blk], step[blk >> 8]));
    const u32x4 w = decode8(codes, t);
    if (r == 0) {                                               // plain dequant, bit for bit (keeps -0)
      *reinterpret_cast<u32x4*>(out + e0) = w;
      continue;
    }
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      o[e] = pack_bf16x2(fmaf(scale, acc[i][2 * e], bf16_lo(w[e])), fmaf(scale, acc[i][2 * e + 1], bf16_hi(w[e])));
    *reinterpret_cast<u32x4*>(out + e0) = u32x4{o[0], o[1], o[2], o[3]};
  }
}

hipError_t launch_merge(const uint8_t* packed, const int8_t* qscale, const float* step, int64_t N, int64_t K,
                        const uint16_t* A, const uint16_t* B, int r, float alpha, uint16_t* out, const Codebook& cb,
                        hipStream_t stream) {
  const int64_t col_chunks = cdiv(K, kMergeCols);
  const int64_t waves = cdiv(N, kMergeRows) * col_chunks;
  const float scale = r > 0 ? alpha / static_cast<float>(r) : 0.0f;
  hipLaunchKernelGGL(k_merge, dim3(static_cast<unsigned>(cdiv(waves, 4))), dim3(256), 0, stream, packed, qscale,
                     step, N, K, A, B, r, scale, out, cb, col_chunks);
  return hipGetLastError();
}

}  // namespace qnf4
