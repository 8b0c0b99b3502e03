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
// kBT: the adapter is B [Kc][r] with r = 16 RT, read in place rather than
// through a transposed copy: each wave copies the B rows of its GS chunks
// (64 rows x 32 RT bytes each, one contiguous run) into its own LDS region
// and reads the operands back with ds_read_b64_tr_b16, whose 16-lane groups
// return one rank column of 4 consecutive rows per lane. The 32-byte pieces
// (row R, rank tile jt) sit at (R RT + jt) ^ bt_swz(R), which keeps both the
// 16-byte copies and the transposed reads (two lane groups per 256-byte
// phase) on 64 distinct banks.
// ---------------------------------------------------------------------------
constexpr int kDownWaves = 8;

template <int RT>
__device__ __forceinline__ int bt_swz(int R) {
  if constexpr (RT == 1) return ((R >> 4) & 1) << 2;
  else if constexpr (RT == 2) return (R >> 4) & 1;
  else if constexpr (RT == 4) return ((R >> 1) & 1) | (((R >> 4) & 1) << 1);
  else return (R & 3) | (((R >> 4) & 1) << 2);
}

template <int RT, int GS, bool kBT>
__global__ __launch_bounds__(64 * kDownWaves) void k_down_rows(const uint16_t* in, int M, int Kc, const uint16_t* W, int r,
                                                   int rp, uint16_t* __restrict__ out, int ldt) {
  // per wave: the staged adapter rows of a round (kBT), then its partial sums
  constexpr int kStage = kBT ? GS * 128 * RT : 0;          // 16-byte chunks
  constexpr int kPer = kStage > 64 * RT ? kStage : 64 * RT;
  __shared__ u32x4 lds[kDownWaves * kPer];
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int m0 = blockIdx.x * 16;
  // uniform by construction; readfirstlane keeps the descriptors in scalar
  // registers (otherwise every load through them becomes a per-lane loop)
  const int rows_valid = __builtin_amdgcn_readfirstlane(M - m0 < 0 ? 0 : (M - m0 < 16 ? M - m0 : 16));
  u32x4* const mine = lds + w * kPer;
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
  // GS chunks per round, all their loads issued before their MFMAs; two
  // rounds in registers, the next one's loads issued before the current one's
  // MFMAs, so each wave keeps a round of loads in flight while it computes
  struct Round {
    u32x4 xa[GS][2];
    u32x4 wv[GS][2 * RT];      // kBT: the B-row pieces; else A rows 16 jt + c, pieces 0 / 1 at 2 jt / 2 jt + 1
  };
  // Loads are issued unconditionally (a conditional round would make the
  // compiler's wait counts assume it missing and drain the pipeline): chunks
  // past the end get an out-of-range offset, which reads zero without a
  // memory access.
  auto load_round = [&](int q0, Round& R) {
#pragma unroll
    for (int u = 0; u < GS; ++u) {
      const int qq = q0 + kDownWaves * u;
      const bool dead = qq >= nchunk;
      const int q = dead ? 0 : qq;
      // wave-uniform; readfirstlane keeps it in a scalar register (a vector
      // soffset turns every load into a per-lane loop)
      const uint32_t so = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(q * 128));
      const uint32_t off_dead = 0x80000000u;
      const uint32_t xv = dead ? off_dead : xo;
      R.xa[u][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, xv, so, 0));
      R.xa[u][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, xv + 16, so, 0));
      if constexpr (kBT) {
        // B rows 64 q .. 64 q + 63: 16-byte piece lane + 64 e of the run
        const uint32_t bo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(q * 2048 * RT));
#pragma unroll
        for (int e = 0; e < 2 * RT; ++e)
          R.wv[u][e] = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, dead ? off_dead : 16 * (lane + 64 * e), bo, 0));
      } else {
#pragma unroll
        for (int jt = 0; jt < RT; ++jt) {
          const uint32_t wv = dead ? off_dead : wo[jt];
          R.wv[u][2 * jt] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, wv, so, 0));
          R.wv[u][2 * jt + 1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, wv + 16, so, 0));
        }
      }
    }
  };
  auto compute_round = [&](int q0, const Round& R) {
    u32x4 wa[GS][RT][2];
    if constexpr (kBT) {
#pragma unroll
      for (int u = 0; u < GS; ++u)
#pragma unroll
        for (int e = 0; e < 2 * RT; ++e) {
          const int pc = lane + 64 * e, sl = pc >> 1, Rw = sl / RT;
          mine[u * 128 * RT + 2 * (sl ^ bt_swz<RT>(Rw)) + (pc & 1)] = R.wv[u][e];
        }
#pragma unroll
      for (int u = 0; u < GS; ++u)
#pragma unroll
        for (int jt = 0; jt < RT; ++jt) {
          s16x4 v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int Rw = 16 * g + 4 * i + (c >> 2);
            v[i] = ds_read_tr(mine + u * 128 * RT, 16 * ((Rw * RT + jt) ^ bt_swz<RT>(Rw)) + 4 * (c & 3));
          }
          wa[u][jt][0] = __builtin_bit_cast(u32x4, __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7));
          wa[u][jt][1] = __builtin_bit_cast(u32x4, __builtin_shufflevector(v[2], v[3], 0, 1, 2, 3, 4, 5, 6, 7));
        }
    } else {
#pragma unroll
      for (int u = 0; u < GS; ++u)
#pragma unroll
        for (int jt = 0; jt < RT; ++jt) {
          wa[u][jt][0] = R.wv[u][2 * jt];
          wa[u][jt][1] = R.wv[u][2 * jt + 1];
        }
    }
#pragma unroll
    for (int u = 0; u < GS; ++u) {
      const int q = q0 + kDownWaves * u;
      const int k = q * 64 + 16 * g;
      // a repeated last chunk, or pieces past Kc, contribute nothing
      const bool live0 = q < nchunk && k < Kc, live1 = q < nchunk && k + 8 < Kc;
      const u32x4 x0 = live0 ? R.xa[u][0] : zero, x1 = live1 ? R.xa[u][1] : zero;
#pragma unroll
      for (int jt = 0; jt < RT; ++jt) {
        acc[jt] = mfma16(as_bf16x8(x0), as_bf16x8(live0 ? wa[u][jt][0] : zero), acc[jt]);
        acc[jt] = mfma16(as_bf16x8(x1), as_bf16x8(live1 ? wa[u][jt][1] : zero), acc[jt]);
      }
    }
  };
  constexpr int kStep = kDownWaves * GS;       // chunks between a wave's rounds
  // two rounds in registers where they fit (RT GS <= 4), else one at a time
  constexpr bool kTwo = RT * GS <= 4;
  Round R0;
  if constexpr (kTwo) {
    Round R1;
    load_round(w, R0);
    // the scheduling barriers keep each round's loads ahead of the MFMAs of
    // the round before it
    for (int q0 = w; q0 < nchunk; q0 += 2 * kStep) {
      const int q1 = q0 + kStep;
      __builtin_amdgcn_sched_barrier(0);
      load_round(q1, R1);
      __builtin_amdgcn_sched_barrier(0);
      compute_round(q0, R0);
      __builtin_amdgcn_sched_barrier(0);
      load_round(q1 + kStep, R0);
      __builtin_amdgcn_sched_barrier(0);
      compute_round(q1, R1);
    }
  } else {
    for (int q0 = w; q0 < nchunk; q0 += kStep) {
      load_round(q0, R0);
      compute_round(q0, R0);
    }
  }
  // the wave's own region takes its partial sums (its last reads of the
  // staged rows come before these writes in its LDS order)
  f32x4* const red = reinterpret_cast<f32x4*>(lds);
#pragma unroll
  for (int jt = 0; jt < RT; ++jt) red[w * kPer + jt * 64 + lane] = acc[jt];
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
      for (int ww = 0; ww < kDownWaves; ++ww) sum += red[ww * kPer + jt * 64 + l][v];
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
  const int nt = down_nt(r);
  if (M > 16) {
    // row-streaming form, no split partials (ldt: the rows up to ldt too);
    // B with r = 16 nt is read in place, other ranks through Bt
    const bool in_place = !wrow && r == 16 * nt;
    const uint16_t* Wr = W;
    if (!wrow && !in_place) {
      hipLaunchKernelGGL(k_adapter_t, dim3(static_cast<unsigned>(cdiv(Kc, 64))), dim3(256), 0, stream, W, Kc, r, wt);
      Wr = wt;
    }
    const unsigned grid16 = static_cast<unsigned>(cdiv(ldt ? ldt : M, 16));
    const int mi = static_cast<int>(M), kci = static_cast<int>(Kc), lt = static_cast<int>(ldt);
    uint16_t* o16 = static_cast<uint16_t*>(out);
#define QNF4_DR(RTV, GSV)                                                                                     \
  do {                                                                                                        \
    if (in_place)                                                                                             \
      hipLaunchKernelGGL(HIP_KERNEL_NAME(k_down_rows<RTV, GSV, true>), dim3(grid16), dim3(64 * kDownWaves), 0, \
                         stream, in, mi, kci, Wr, r, rp, o16, lt);                                            \
    else                                                                                                      \
      hipLaunchKernelGGL(HIP_KERNEL_NAME(k_down_rows<RTV, GSV, false>), dim3(grid16), dim3(64 * kDownWaves), 0, \
                         stream, in, mi, kci, Wr, r, rp, o16, lt);                                            \
  } while (0)
    if (nt == 1)
      QNF4_DR(1, 4);
    else if (nt == 2)
      QNF4_DR(2, 2);
    else if (nt == 4)
      QNF4_DR(4, 1);
    else
      QNF4_DR(8, 1);
#undef QNF4_DR
    return hipGetLastError();
  }
  const uint16_t* Wr = W;
  if (!wrow) {
    hipLaunchKernelGGL(k_adapter_t, dim3(static_cast<unsigned>(cdiv(Kc, 64))), dim3(256), 0, stream, W, Kc, r, wt);
    Wr = wt;
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
