// Merge of the LoRA adapter into one dense bf16 weight for deployment: the
// update is the usual low-rank one, so it folds back into the weights ("QLoRA"
// (techbytebybyte), "Curiosity question: is the final model permanently
// 4-bit?" and "Training setup versus deployment setup"; "A 65B fine-tune on
// the GPU you already have", figure 2):
//     out[n][k] = bf16( W'[n][k] + (alpha / r) . sum_j B[n][j] . A[j][k] )
// with W' the dequantized bf16 weight (the exact arithmetic of
// qlora_nf4_dequant). The rank-r sum is a bf16 x bf16 product accumulated in
// fp32, then one fused multiply-add with the scale onto W' and one rounding to
// bf16. Without an adapter the output is the dequantized weight, bit for bit.
//
// k_merge: a workgroup owns a 16 x 256 (ranks up to 32) or 32 x 256 output
// tile (the staged slice of A is then shared by more rows). The rank-r sum is an MFMA
// contraction over the ranks (16x16x32 bf16, ranks padded to 32 with zeros),
// computed transposed, so that a lane's four results are four consecutive
// columns of one row: the A operands are A's columns (8 ranks of one column),
// read transposed (ds_read_b64_tr_b16) from the tile's rp x 256 slice of A
// staged once in LDS, the B operands B's rows (8 consecutive ranks of one row,
// one 16-byte load); wave w computes columns 64w .. 64w + 63 of all rows.
// The fp32 tile goes through LDS (16-byte chunks, row-swizzled) to rows of 8
// consecutive columns, where each lane decodes one packed code dword with its
// block's table, adds, rounds and stores 16 bytes. The code words and block
// scales are requested before the contraction, so their loads overlap it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mm_common.hpp"

namespace qnf4 {

namespace {
constexpr int kMgCols = 256;              // output columns per workgroup
// output rows per workgroup for RC rank chunks of 32
constexpr int mg_rows(int rc) { return rc <= 1 ? 16 : 32; }

// chunk q (0..31) of rank row j of the staged A slice: the transposed reads
// (32 lanes: ranks R .. R+3 and R+8 .. R+11, two adjacent chunks) touch all 64
// banks once
__device__ __forceinline__ int mg_slot(int j, int q) {
  return j * 32 + (q ^ (2 * ((j & 3) | (((j >> 3) & 1) << 2))));
}
}  // namespace

// RC: rank chunks of 32 (rank_pad(r) / 32), 0 for no adapter.
template <int RC>
__global__ __launch_bounds__(256) void k_merge(const uint8_t* __restrict__ packed, const int8_t* __restrict__ qscale,
                                               const float* __restrict__ step, int64_t N, int64_t K,
                                               const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, int r,
                                               float scale, uint16_t* __restrict__ out, Codebook cb, int64_t ktiles) {
  // A's slice (32 RC rank rows x 32 chunks), then the fp32 tile
  // [kMgRows][256] (64 chunks of 16 bytes per row, chunk q of row n at
  // q ^ (n % 16))
  constexpr int kMgRows = mg_rows(RC);
  constexpr int kMgGroups = kMgRows * kMgCols / 8 / 256;   // 8-column groups per thread
  constexpr int kSChunks = 32 * RC * 32 > kMgRows * kMgCols / 4 ? 32 * RC * 32 : kMgRows * kMgCols / 4;
  __shared__ u32x4 S[RC > 0 ? kSChunks : 1];
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int64_t n0 = (static_cast<int64_t>(blockIdx.x) / ktiles) * kMgRows;
  const int64_t k0 = (static_cast<int64_t>(blockIdx.x) % ktiles) * kMgCols;

  // thread t's output groups gi = t + 256 i: row gi / 32, columns 8 (gi % 32)
  // .. + 7 (32 threads cover one row's 256 columns: 128 code bytes in, 512
  // output bytes out); their code words and block scales, requested first
  uint32_t codes[kMgGroups];
  float sc[kMgGroups];
#pragma unroll
  for (int i = 0; i < kMgGroups; ++i) {
    const int gi = 256 * i + t;
    const int64_t n = n0 + (gi >> 5), k = k0 + 8 * (gi & 31);
    const bool in = n < N && k < K;
    const int64_t e0 = in ? n * K + k : 0;
    codes[i] = in ? *reinterpret_cast<const uint32_t*>(packed + e0 / 2) : 0u;
    sc[i] = in ? block_scale(qscale[e0 / 64], step[e0 / 16384]) : 0.0f;
  }

  if constexpr (RC > 0) {
    // A[j][k0 .. k0 + 255] for j < 32 RC (zero past r or K)
    for (int i = t; i < 32 * RC * 32; i += 256) {
      const int j = i >> 5, q = i & 31;
      const int64_t kk = k0 + 8 * q;
      S[mg_slot(j, q)] = (j < r && kk < K) ? ld16(A + static_cast<int64_t>(j) * K + kk) : u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
    // wave w, lane (g, c) of tile (cb, rb): row 16rb + c, columns
    // 64w + 16cb + 4g .. + 3
    f32x4 acc[kMgRows / 16][4];
#pragma unroll
    for (int rb = 0; rb < kMgRows / 16; ++rb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) acc[rb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int rc = 0; rc < RC; ++rc) {
      // B operands: B[n0 + 16rb + c][32rc + 8g .. + 7] (zero past N or r)
      u32x4 bo[kMgRows / 16];
#pragma unroll
      for (int rb = 0; rb < kMgRows / 16; ++rb) {
        const int64_t n = n0 + 16 * rb + c;
        const int j0 = 32 * rc + 8 * g;
        if ((r & 7) == 0) {
          bo[rb] = (n < N && j0 < r) ? ld16(B + n * r + j0) : u32x4{0u, 0u, 0u, 0u};
        } else {                                   // rows of B not 16-byte aligned: one rank at a time
          uint32_t v[4] = {0u, 0u, 0u, 0u};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t h = (n < N && j0 + e < r) ? static_cast<uint32_t>(B[n * r + j0 + e]) : 0u;
            v[e >> 1] |= h << (16 * (e & 1));
          }
          bo[rb] = u32x4{v[0], v[1], v[2], v[3]};
        }
      }
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        // A operand: ranks 32rc + 8g .. + 7 of column 64w + 16cb + c, as two
        // transposed reads (ranks + 4q + c/4, columns + 4 (c % 4) .. + 3)
        s16x4 v[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int j = 32 * rc + 8 * g + 4 * q + (c >> 2), col = 64 * w + 16 * cb + 4 * (c & 3);
          v[q] = ds_read_tr(S, mg_slot(j, col >> 3) * 8 + (col & 4));
        }
        const bf16x8 ao = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int rb = 0; rb < kMgRows / 16; ++rb) acc[rb][cb] = mfma16(ao, as_bf16x8(bo[rb]), acc[rb][cb]);
      }
    }
    __syncthreads();                               // A's slice is read: the memory takes the fp32 tile
#pragma unroll
    for (int rb = 0; rb < kMgRows / 16; ++rb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int row = 16 * rb + c, q = 16 * w + 4 * cb + g;
        S[row * 64 + (q ^ c)] = __builtin_bit_cast(u32x4, acc[rb][cb]);
      }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < kMgGroups; ++i) {
    const int gi = 256 * i + t, row = gi >> 5, grp = gi & 31;
    const int64_t n = n0 + row, k = k0 + 8 * grp;
    if (n >= N || k >= K) continue;
    const u32x4 wv = decode8(codes[i], make_table(cb, sc[i]));
    uint16_t* const o = out + n * K + k;
    if constexpr (RC == 0) {                                    // plain dequant, bit for bit (keeps -0)
      *reinterpret_cast<u32x4*>(o) = wv;
    } else {
      const f32x4 s0 = __builtin_bit_cast(f32x4, S[row * 64 + ((2 * grp) ^ (row & 15))]);
      const f32x4 s1 = __builtin_bit_cast(f32x4, S[row * 64 + ((2 * grp + 1) ^ (row & 15))]);
      const float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
      uint32_t ov[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        ov[e] = pack_bf16x2(fmaf(scale, sv[2 * e], bf16_lo(wv[e])), fmaf(scale, sv[2 * e + 1], bf16_hi(wv[e])));
      *reinterpret_cast<u32x4*>(o) = u32x4{ov[0], ov[1], ov[2], ov[3]};
    }
  }
}

hipError_t launch_merge(const uint8_t* packed, const int8_t* qscale, const float* step, int64_t N, int64_t K,
                        const uint16_t* A, const uint16_t* B, int r, float alpha, uint16_t* out, const Codebook& cb,
                        hipStream_t stream) {
  const int64_t ktiles = cdiv(K, kMgCols);
  const float scale = r > 0 ? alpha / static_cast<float>(r) : 0.0f;
  const int rc = r > 0 ? static_cast<int>(rank_pad(r) / 32) : 0;
#define QNF4_MG(RCV)                                                                                         \
  hipLaunchKernelGGL(k_merge<RCV>, dim3(static_cast<unsigned>(cdiv(N, mg_rows(RCV)) * ktiles)), dim3(256), 0, \
                     stream, packed, qscale, step, N, K, A, B, r, scale, out, cb, ktiles)
  switch (rc) {
    case 0: QNF4_MG(0); break;
    case 1: QNF4_MG(1); break;
    case 2: QNF4_MG(2); break;
    case 3: QNF4_MG(3); break;
    default: QNF4_MG(4); break;
  }
#undef QNF4_MG
  return hipGetLastError();
}

}  // namespace qnf4
