// Decode-shaped (M <= 16) fused NF4-dequant backward for gfx950.
//
// At these shapes every weight is used by at most 16 rows, so the kernels are
// bound by streaming the 0.516 bytes/param NF4 weight from HBM. Operands of
// the next step are loaded while the current one is decoded and multiplied.
//
//   k_bwd_small   dX partials: 64-column tiles x row slices; 1024 weight rows
//                 per step dequantized into LDS and read transposed
//                 (ds_read_b64_tr_b16).
//   k_bwd_finish  dX = bf16(sum of the row-slice partials + LoRA term).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mm_common.hpp"

namespace qnf4 {

// ---------------------------------------------------------------------------
// k_bwd_small: grid (K/64 column tiles, S row slices), 16 waves. Each step
// dequantizes 1024 weight rows x one 64-column block (one block per thread)
// into LDS; wave w contracts rows [64w, 64w + 64) of the step on 16x16x32
// MFMAs with the B operand read transposed. The LDS tile is reused for the
// cross-wave reduction.
// ---------------------------------------------------------------------------
constexpr int kBwdWaves = 16;
constexpr int kBwdRows = 64 * kBwdWaves;       // weight rows per step

__device__ __forceinline__ int sm_slot(int row, int ch) {
  // 8 consecutive rows writing one chunk hit 8 bank groups; the 4 rows one
  // transposed read touches get 4 distinct chunk pairs
  const int sw = ((row & 3) << 1) | ((row >> 2) & 1);
  return row * 8 + (ch ^ sw);
}

// Workgroup id -> (column tile kt, row slice s). A 128-byte line of a packed
// weight row holds the codes of four consecutive column tiles; the four
// workgroups that share it are given consecutive ids on one XCD (ids go
// round-robin over the 8 XCDs), so the line is fetched into that XCD's L2
// once instead of once per tile.
__device__ __forceinline__ void bwd_tile_of(int lin, int ktiles, int S, int& kt, int& s) {
  if ((ktiles & 3) == 0 && ((ktiles * S) & 31) == 0) {
    const int xcd = lin & 7, j = lin >> 3;
    const int p = 8 * (j >> 2) + xcd;
    kt = 4 * (p % (ktiles >> 2)) + (j & 3);
    s = p / (ktiles >> 2);
  } else {
    kt = lin % ktiles;
    s = lin / ktiles;
  }
}

// The workgroups of column tile 0 also compute this slice's share of the LoRA
// down-projection u = dY . B (B [N][r]), from the same dY fragments:
// upart[s][m][rp] fp32, summed over slices by k_bwd_finish. NTU: rank tiles
// of 16 (ceil(r / 16), rounded up to a power of two; 0 without an adapter).
template <int NTU>
__global__ __launch_bounds__(64 * kBwdWaves) void k_bwd_small(const uint16_t* __restrict__ dy, int64_t M,
                                                              int64_t N, int64_t K,
                                                              const uint8_t* __restrict__ packed,
                                                              const int8_t* __restrict__ qscale,
                                                              const float* __restrict__ step, int S,
                                                              float* __restrict__ part,
                                                              const uint16_t* __restrict__ Bl, int r, int rp,
                                                              float* __restrict__ upart, Codebook cb) {
  __shared__ u32x4 Bs[kBwdRows * 8];         // 128 KB: one step's tile, then the reduction
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  int kti, s;
  bwd_tile_of(blockIdx.x, static_cast<int>(K / 64), S, kti, s);
  const int64_t kt = kti;                    // 64-column tile == block column kt
  const bool do_u = kti == 0 && r > 0;
  const int ntu = do_u ? (r + 15) / 16 : 0;  // rank tiles of u computed here (<= NTU)
  const int64_t nbr = K / 64;
  const int64_t nsteps = cdiv(N, kBwdRows);
  const int64_t st_beg = s * nsteps / S, st_end = (s + 1) * nsteps / S;
  const int64_t m = imin(static_cast<int64_t>(lane & 15), M - 1);
  const int G = lane >> 4, j16 = lane & 15;
  constexpr int kU = NTU > 0 ? NTU : 1;
  f32x4 acc[4], uacc[kU];
#pragma unroll
  for (int cbk = 0; cbk < 4; ++cbk) acc[cbk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int jt = 0; jt < kU; ++jt) uacc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int64_t st = st_beg; st < st_end; ++st) {
    // this thread's weight row-block and this wave's dY fragments
    const int64_t row = imin(st * kBwdRows + t, N - 1);
    const uint8_t* p = packed + row * (K / 2) + kt * 32;
    const u32x4 b0 = ld16(p), b1 = ld16(p + 16);
    const int64_t blk = row * nbr + kt;
    const int8_t qv = qscale[blk];
    const float dv = step[blk >> 8];
    u32x4 av[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int64_t ncol = st * kBwdRows + 64 * w + 32 * ks + 8 * G;
      av[ks] = ncol < N ? ld16(dy + m * N + ncol) : u32x4{0u, 0u, 0u, 0u};
    }
    if (st > st_beg) __syncthreads();        // previous step's reads are done
    {
      const MagTable tb = make_table(cb, block_scale(qv, dv));
      const uint32_t pw[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
      for (int ch = 0; ch < 8; ++ch) Bs[sm_slot(t, ch)] = decode8(pw[ch], tb);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int cbk = 0; cbk < 4; ++cbk) {
        const int col = 16 * cbk + 4 * (j16 & 3);
        s16x4 v[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int rr = 64 * w + 32 * ks + 8 * G + 4 * q + (j16 >> 2);
          v[q] = ds_read_tr(Bs, sm_slot(rr, col >> 3) * 8 + (col & 4));
        }
        const bf16x8 bv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7));
        acc[cbk] = mfma16(as_bf16x8(av[ks]), bv, acc[cbk]);
      }
    }
    if (NTU > 0 && do_u) {
      // B operand of u: lane (rank 16 jt + j16, rows n0 .. n0 + 7 of the
      // contraction) from B [N][r], zero past N or r
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int64_t n0 = st * kBwdRows + 64 * w + 32 * ks + 8 * G;
#pragma unroll
        for (int jt = 0; jt < NTU; ++jt) {
          if (jt < ntu) {
            const int j = 16 * jt + j16;
            uint32_t bv[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int64_t n = n0 + e;
              const uint32_t val = (n < N && j < r) ? static_cast<uint32_t>(Bl[n * r + j]) : 0u;
              bv[e >> 1] |= val << (16 * (e & 1));
            }
            uacc[jt] = mfma16(as_bf16x8(av[ks]), as_bf16x8(u32x4{bv[0], bv[1], bv[2], bv[3]}), uacc[jt]);
          }
        }
      }
    }
  }
  __syncthreads();                             // tile reads done: reuse LDS
  f32x4* red = reinterpret_cast<f32x4*>(Bs);   // [wave][cbk][lane]
#pragma unroll
  for (int cbk = 0; cbk < 4; ++cbk) red[(w * 4 + cbk) * 64 + lane] = acc[cbk];
  __syncthreads();
  if (t < 256) {
    const int cbk = t >> 6, ln = t & 63;
    f32x4 sum = red[cbk * 64 + ln];
#pragma unroll
    for (int i = 1; i < kBwdWaves; ++i) sum += red[(i * 4 + cbk) * 64 + ln];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t mm = 4 * (ln >> 4) + v;
      if (mm < M) part[(s * M + mm) * K + kt * 64 + 16 * cbk + (ln & 15)] = sum[v];
    }
  }
  if (NTU > 0 && do_u) {
    // u partials of this slice: lane (G, j16) of tile jt holds u[4 G + v][16 jt + j16]
    __syncthreads();
#pragma unroll
    for (int jt = 0; jt < NTU; ++jt)
      if (jt < ntu) red[(w * 8 + jt) * 64 + lane] = uacc[jt];
    __syncthreads();
    for (int idx = t; idx < ntu * 64; idx += 64 * kBwdWaves) {
      const int jt = idx >> 6, ln = idx & 63;
      f32x4 sum = red[jt * 64 + ln];
#pragma unroll
      for (int i = 1; i < kBwdWaves; ++i) sum += red[(i * 8 + jt) * 64 + ln];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t mm = 4 * (ln >> 4) + v;
        if (mm < M) upart[(s * M + mm) * rp + 16 * jt + (ln & 15)] = sum[v];
      }
    }
    // ranks between ceil(r/16)*16 and rp are zero
    for (int idx = t; idx < M * rp; idx += 64 * kBwdWaves) {
      const int rank = idx % rp;
      if (rank >= 16 * ntu) upart[s * M * rp + idx] = 0.0f;
    }
  }
}

// dX[m][k] = bf16( sum_s part[s][m][k] + scale * sum_j u[m][j] A[j][k] ),
// u = bf16(sum of the down-projection partials). Grid (ceil(K/256), M).
__global__ __launch_bounds__(256) void k_bwd_finish(const float* __restrict__ part, int S, int64_t M, int64_t K,
                                                    const float* __restrict__ upart, int Su, int rp,
                                                    const uint16_t* __restrict__ Al, int r, float scale,
                                                    uint16_t* __restrict__ dx) {
  __shared__ float us[128];
  const int t = threadIdx.x;
  const int64_t m = blockIdx.y;
  const int64_t k = static_cast<int64_t>(blockIdx.x) * 256 + t;
  const int64_t kc = imin(k, K - 1);
  float v = 0.f;
  for (int s = 0; s < S; ++s) v += part[(s * M + m) * K + kc];
  if (r > 0) {
    // this column of A, loaded before the barrier (ranks beyond 32 after it)
    float av[32];
#pragma unroll
    for (int j = 0; j < 32; ++j)
      av[j] = j < r ? bf16_lo(static_cast<uint32_t>(Al[static_cast<int64_t>(j) * K + kc])) : 0.0f;
    if (t < rp) {
      float u = 0.f;
      for (int s = 0; s < Su; ++s) u += upart[(s * M + m) * rp + t];
      us[t] = bf16_lo(static_cast<uint32_t>(bf16_bits(u)));
    }
    __syncthreads();
    float l = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) l += us[j < rp ? j : 0] * av[j];
    for (int j = 32; j < r; ++j) l += us[j] * bf16_lo(static_cast<uint32_t>(Al[static_cast<int64_t>(j) * K + kc]));
    v += scale * l;
  }
  if (k < K) dx[m * K + k] = bf16_bits(v);
}

// ---------------------------------------------------------------------------
// launchers (M <= 16)
// ---------------------------------------------------------------------------
hipError_t launch_bwd_small(const uint16_t* dy, int64_t M, int64_t N, int64_t K, const uint8_t* packed,
                            const int8_t* qscale, const float* step, float* upart, int rp, const uint16_t* A,
                            const uint16_t* B, int r, float scale, float* part, uint16_t* dx, const Codebook& cb,
                            hipStream_t stream) {
  const int S = static_cast<int>(bwd_small_splits(N, K));
  const dim3 grid(static_cast<unsigned>((K / 64) * S)), block(64 * kBwdWaves);
  const int nt = r > 0 ? (r + 15) / 16 : 0;
#define QNF4_BWDS(NTV)                                                                                        \
  hipLaunchKernelGGL(k_bwd_small<NTV>, grid, block, 0, stream, dy, M, N, K, packed, qscale, step, S, part, B, r, \
                     rp, upart, cb)
  mark_kernel(0, stream);
  if (nt == 0)
    QNF4_BWDS(0);
  else if (nt == 1)
    QNF4_BWDS(1);
  else if (nt == 2)
    QNF4_BWDS(2);
  else if (nt <= 4)
    QNF4_BWDS(4);
  else
    QNF4_BWDS(8);
#undef QNF4_BWDS
  mark_kernel(1, stream);
  hipLaunchKernelGGL(k_bwd_finish, dim3(static_cast<unsigned>(cdiv(K, 256)), static_cast<unsigned>(M)), dim3(256),
                     0, stream, part, S, M, K, upart, S, rp, A, r, scale, dx);
  return hipGetLastError();
}

}  // namespace qnf4
