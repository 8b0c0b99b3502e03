// Fused NF4-dequant matmuls for gfx950 (MI355X).
//
// Forward  y  = bf16( x . W'^T + (alpha/r) . t . B^T ),  t = bf16(x . A^T)
// Backward dX = bf16( dY . W'  + (alpha/r) . u . A   ),  u = bf16(dY . B)
// with W' the bf16 dequantization of the NF4 weight, done block by block
// right before the multiply ("A 65B fine-tune on the GPU you already have",
// figure 2; "QLoRA Explained", "What is QLoRA?").
//
// Kernels
//   k_lora_down   rank-r down projection (t or u) on 16x16x32 bf16 MFMA.
//   k_gemv_fwd    M <= 16: 16 weight rows per workgroup, 8 waves splitting K;
//                 each lane dequantizes one 64-block straight into the MFMA
//                 B-operand registers (no LDS); HBM-bound.
//   k_gemm_fwd    M > 16: 256x256 output tile, 4 waves each owning 64 output
//                 columns; each lane dequantizes its MFMA B operands straight
//                 into registers, x goes through double-buffered LDS; 32x32x16
//                 bf16 MFMA with fp32 accumulation; LoRA as a rank-r MFMA in
//                 the epilogue. MFMA-bound.
//   k_gemm_bwd    M > 16: same tiling over dX [M, K]; the contraction runs over
//                 W's rows, so the dequantized tile is stored row-major and
//                 read transposed with ds_read_b64_tr_b16.
//   k_bwd_small   M <= 16 backward: 64-column tiles, row slices reduced by
//   k_bwd_finish  a second kernel that also adds the LoRA term.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mm_common.hpp"

namespace qnf4 {

// ---------------------------------------------------------------------------
// Tiled MFMA GEMMs (M > 16)
// ---------------------------------------------------------------------------
constexpr int kTile = 256;
constexpr int kChunks = 2048;                // 16-byte chunks in one 256x64 bf16 tile

// Workgroup id -> output tile. Consecutive ids land on different XCDs (round
// robin over 8), so each XCD is first given a contiguous range of the tile
// order; that order then sweeps groups of 8 tile-rows across all tile-columns
// so co-resident workgroups share operand tiles in their XCD's L2.
__device__ __forceinline__ void tile_of(int pid, int ntm, int ntn, int& tm, int& tn) {
  const int total = ntm * ntn;
  int p = pid;
  if ((total & 7) == 0) p = (pid & 7) * (total >> 3) + (pid >> 3);
  const int G = 8;
  const int group = p / (G * ntn);
  const int first_m = group * G;
  const int gsz = (ntm - first_m) < G ? (ntm - first_m) : G;
  const int within = p - group * G * ntn;
  tm = first_m + within % gsz;
  tn = within / gsz;
}

// A tile (256 rows x 64 deep, bf16) in LDS: row-major, 8 chunks of 16 bytes
// per row, chunk index xor (row & 7) so that 8 consecutive rows reading the
// same logical chunk hit 8 different bank groups.
__device__ __forceinline__ int a_slot(int row, int ch) { return row * 8 + (ch ^ (row & 7)); }

// ---------------------------------------------------------------------------
// k_gemm_fwd: y [M, N] = x . W'^T (+ LoRA), M > 16.
//
// Workgroup tile 256 (M) x 256 (N), 4 waves; wave w owns output columns
// [64w, 64w + 64) for all 256 rows: 8 x 2 blocks of 32x32x16 bf16 MFMA with
// fp32 accumulators. In this NT layout one packed dword (8 codes of one
// weight row) is exactly one MFMA B operand, so each lane dequantizes its own
// B operands straight into registers: no LDS for the weights and every weight
// decoded once. x goes global -> LDS directly (global_load_lds_dwordx4: lane i
// of a wave lands at LDS base + 16 i, so the bank swizzle is applied on the
// global side), double-buffered.
//
// Per 64-deep K step k: packed codes of step k+2 are loaded into registers,
// the MFMAs of step k run while the codes of step k+1 are decoded, and after
// the barrier that ends the step the x tile of step k+2 is requested. Every
// load thus has a whole step to land, and the loop (unrolled by two) keeps its
// register sets fixed.
//
// K permutation: within a step, lane half h holds k in [32h, 32h + 32) and
// MFMA sub-step s uses k = 32h + 8s + (0..7) on both operands (the sum over k
// is order-free), so a lane's codes for a step are one 16-byte load.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

struct BPacked {
  u32x4 p[2];      // packed codes of this lane's weight row, N-block j
  float d[2];
  int8_t q[2];
};

// s_waitcnt vmcnt(0) (expcnt/lgkmcnt untouched), as the builtin so the
// compiler's own wait insertion knows every earlier load has completed
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__global__ __launch_bounds__(256, 1) void k_gemm_fwd(const uint16_t* __restrict__ x, int64_t M, int64_t N,
                                                     int64_t K, const uint8_t* __restrict__ packed,
                                                     const int8_t* __restrict__ qscale,
                                                     const float* __restrict__ step,
                                                     const uint16_t* __restrict__ tl, int rp,
                                                     const uint16_t* __restrict__ Bl, int r, float scale,
                                                     uint16_t* __restrict__ y, Codebook cb) {
  __shared__ u32x4 As0[kChunks];             // two distinct 32 KB buffers, so the
  __shared__ u32x4 As1[kChunks];             // compiler can tell a DMA into one from reads of the other
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int ntm = static_cast<int>(cdiv(M, kTile)), ntn = static_cast<int>(cdiv(N, kTile));
  int tm, tn;
  tile_of(blockIdx.x, ntm, ntn, tm, tn);
  const int64_t m0 = static_cast<int64_t>(tm) * kTile, n0 = static_cast<int64_t>(tn) * kTile;
  const int64_t nk = K / 64;

  // x tile DMA: instruction i of wave w fills LDS rows 64w + 8i + (lane >> 3),
  // physical chunk lane & 7, i.e. logical chunk (lane & 7) ^ (lane >> 3)
  const int dchunk = (lane & 7) ^ (lane >> 3);
  const uint16_t* aptr[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) aptr[i] = x + imin(m0 + 64 * w + 8 * i + (lane >> 3), M - 1) * K + 8 * dchunk;
  auto dma_a = [&](int64_t kt, u32x4* Ab) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      lds_void* dst = (lds_void*)(&Ab[(64 * w + 8 * i) * 8]);
      __builtin_amdgcn_global_load_lds((gbl_void*)(aptr[i] + kt * 64), dst, 16, 0, 0);
    }
  };
  const uint8_t* bptr[2];
  int64_t bblk[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t n = imin(n0 + 64 * w + 32 * j + l32, N - 1);
    bptr[j] = packed + n * (K / 2) + 16 * h;
    bblk[j] = n * nk;
  }
  auto load_b = [&](int64_t kt, BPacked& P) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      P.p[j] = ld16(bptr[j] + kt * 32);
      P.q[j] = qscale[bblk[j] + kt];
      P.d[j] = step[(bblk[j] + kt) >> 8];
    }
  };
  f32x16 acc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // MFMAs of one step (A buffer `buf`, decoded B `bo`) with the decode of the
  // next step's codes `nx` into `bn` spread over the four sub-steps.
  auto step_k = [&](const u32x4* Ab, u32x4* An, const bf16x8 (&bo)[2][4], const BPacked& nx,
                    bf16x8 (&bn)[2][4], int64_t kload, BPacked& ld, int64_t kdma) {
    dma_a(kdma, An);
    load_b(kload, ld);
    __builtin_amdgcn_sched_barrier(0);         // keep this step's loads at its head
    MagTable tb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) tb[j] = make_table(cb, block_scale(nx.q[j], nx.d[j]));
    // A fragments double-buffered across sub-steps: those of s+1 are read
    // while the MFMAs of s issue
    bf16x8 afr[2][8];
    auto read_frags = [&](int s, bf16x8 (&af)[8]) {
      const int sw = (4 * h + s) ^ (l32 & 7);
#pragma unroll
      for (int i = 0; i < 8; ++i) af[i] = as_bf16x8(Ab[(32 * i + l32) * 8 + sw]);
    };
    read_frags(0, afr[0]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) read_frags(s + 1, afr[(s + 1) & 1]);
      const bf16x8 (&af)[8] = afr[s & 1];
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[i], bo[j][s], acc[i][j]);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t pw = s == 0 ? nx.p[j].x : s == 1 ? nx.p[j].y : s == 2 ? nx.p[j].z : nx.p[j].w;
        bn[j][s] = as_bf16x8(decode8(pw, tb[j]));
      }
    }
    // issue order after the loads: the A fragments of sub-step 0, then each
    // MFMA followed by four VALU ops (the decode of the next step) and, every
    // other MFMA, one LDS read of the next sub-step's A fragments
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int m = 0; m < 64; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if ((m & 1) == 0 && m < 48) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    }
  };
  auto decode_all = [&](const BPacked& P, bf16x8 (&bo)[2][4]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const MagTable tb = make_table(cb, block_scale(P.q[j], P.d[j]));
      bo[j][0] = as_bf16x8(decode8(P.p[j].x, tb));
      bo[j][1] = as_bf16x8(decode8(P.p[j].y, tb));
      bo[j][2] = as_bf16x8(decode8(P.p[j].z, tb));
      bo[j][3] = as_bf16x8(decode8(P.p[j].w, tb));
    }
  };

  BPacked P0, P1;
  bf16x8 B0[2][4], B1[2][4];
  dma_a(0, As0);
  load_b(0, P0);
  load_b(imin(1, nk - 1), P1);
  __builtin_amdgcn_sched_barrier(0);
  wait_vm0();
  // pin step 1's codes here: left alone, the (read-only) loads get sunk into
  // the loop entry, and the loop head would then drain every later load
  asm volatile("" ::"v"(P1.p[0]), "v"(P1.p[1]), "v"(static_cast<int>(P1.q[0])), "v"(static_cast<int>(P1.q[1])),
               "v"(P1.d[0]), "v"(P1.d[1]));
  decode_all(P0, B0);
  __syncthreads();
  int64_t kt = 0;
  // step kt reads A buffer kt%2 while the x tile of kt+1 streams into the
  // other buffer (requested at the start of the step, after the barrier that
  // ended step kt-1, which was the last reader of that buffer)
  for (; kt + 2 <= nk; kt += 2) {
    step_k(As0, As1, B0, P1, B1, imin(kt + 2, nk - 1), P0, imin(kt + 1, nk - 1));
    wait_vm0();
    __syncthreads();
    step_k(As1, As0, B1, P0, B0, imin(kt + 3, nk - 1), P1, imin(kt + 2, nk - 1));
    wait_vm0();
    __syncthreads();
  }
  if (kt < nk) step_k(As0, As1, B0, P1, B1, nk - 1, P0, nk - 1);
  wait_vm0();

  // epilogue: LoRA up-projection as a rank-r MFMA, then bf16 stores
  if (r > 0) {
    const bool vec_ok = (r & 7) == 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t mrow = imin(m0 + 32 * i + l32, M - 1);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t nrow = imin(n0 + 64 * w + 32 * j + l32, N - 1);
        f32x16 tmp;
#pragma unroll
        for (int v = 0; v < 16; ++v) tmp[v] = 0.f;
        for (int rs = 0; rs < rp / 16; ++rs) {
          const bf16x8 a = as_bf16x8(ld16(tl + mrow * rp + 16 * rs + 8 * h));
          const bf16x8 b = as_bf16x8(load_row8(Bl + nrow * r, 16 * rs + 8 * h, r, vec_ok));
          tmp = mfma32(a, b, tmp);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] += scale * tmp[v];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t nn = n0 + 64 * w + 32 * j + l32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t mm = m0 + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
        if (mm < M && nn < N) y[mm * N + nn] = bf16_bits(acc[i][j][v]);
      }
    }
}

// B tile of the backward: 64 weight rows x 256 output columns, bf16, 32
// chunks per row. Within each 8-chunk (64-column) group the chunk index is
// xor-ed with g(row, group): bits 2..1 separate 4 consecutive rows (the rows
// one transposed read touches) and bit 0 separates neighbouring rows, which
// keeps both the producer's 16-byte writes and the 8-byte transposed reads
// spread over the banks.
__device__ __forceinline__ int bw_slot(int row, int ch) {
  const int grp = ch >> 3;
  const int g = ((((row & 3) ^ grp) & 3) << 1) | (row & 1);
  return row * 32 + (ch ^ g);
}

__global__ __launch_bounds__(256, 1) void k_gemm_bwd(const uint16_t* __restrict__ dy, int64_t M, int64_t N,
                                                     int64_t K, const uint8_t* __restrict__ packed,
                                                     const int8_t* __restrict__ qscale,
                                                     const float* __restrict__ step,
                                                     const uint16_t* __restrict__ ul, int rp,
                                                     const uint16_t* __restrict__ Al, int r, float scale,
                                                     uint16_t* __restrict__ dx, Codebook cb) {
  __shared__ u32x4 smem[4 * kChunks];
  u32x4* As = smem;
  u32x4* Bs = smem + 2 * kChunks;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int h = lane >> 5, l32 = lane & 31;
  const int ntm = static_cast<int>(cdiv(M, kTile)), ntk = static_cast<int>(cdiv(K, kTile));
  int tm, tk;
  tile_of(blockIdx.x, ntm, ntk, tm, tk);
  const int64_t m0 = static_cast<int64_t>(tm) * kTile, k0 = static_cast<int64_t>(tk) * kTile;
  const int64_t nbr = K / 64;
  const int64_t nsteps = cdiv(N, 64);

  // A (dY) staging: row arow0 + 32i, contraction chunk ach
  const int ach = t & 7, arow0 = t >> 3;
  const uint16_t* aptr[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) aptr[i] = dy + imin(m0 + arow0 + 32 * i, M - 1) * N + ach * 8;
  // B staging: weight row nn of the step, 64-column group kb of the tile
  const int bnn = t >> 2, bkb = t & 3;
  const int64_t bkbi = imin(k0 / 64 + bkb, nbr - 1);

  u32x4 areg[8];
  u32x4 b0, b1;
  int8_t qv;
  float dv;
  auto gload = [&](int64_t st) {
    const int64_t nbase = st * 64;
    const bool aval = nbase + ach * 8 < N;
#pragma unroll
    for (int i = 0; i < 8; ++i) areg[i] = aval ? ld16(aptr[i] + nbase) : u32x4{0u, 0u, 0u, 0u};
    const int64_t row = imin(nbase + bnn, N - 1);
    const uint8_t* p = packed + row * (K / 2) + bkbi * 32;
    b0 = ld16(p);
    b1 = ld16(p + 16);
    const int64_t blk = row * nbr + bkbi;
    qv = qscale[blk];
    dv = step[blk >> 8];
  };
  auto lstore = [&](int buf) {
    u32x4* Ab = As + buf * kChunks;
    u32x4* Bb = Bs + buf * kChunks;
#pragma unroll
    for (int i = 0; i < 8; ++i) Ab[a_slot(arow0 + 32 * i, ach)] = areg[i];
    const MagTable tb = make_table(cb, block_scale(qv, dv));
    const uint32_t pw[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) Bb[bw_slot(bnn, 8 * bkb + ch)] = decode8(pw[ch], tb);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int G = lane >> 4, j16 = lane & 15;
  const int hh = G >> 1, cbh = G & 1;
  auto compute = [&](int buf) {
    const u32x4* Ab = As + buf * kChunks;
    const u32x4* Bb = Bs + buf * kChunks;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int sw = (2 * ks + h) ^ (l32 & 7);
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = as_bf16x8(Ab[(128 * wm + 32 * i + l32) * 8 + sw]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = 128 * wn + 32 * j + 16 * cbh + 4 * (j16 & 3);
        s16x4 v[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int row = 16 * ks + 8 * hh + 4 * q + (j16 >> 2);
          v[q] = ds_read_tr(Bb, bw_slot(row, col >> 3) * 8 + (col & 4));
        }
        bfr[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
  };

  gload(0);
  lstore(0);
  __syncthreads();
  for (int64_t st = 0; st < nsteps; ++st) {
    const int cur = static_cast<int>(st & 1);
    const bool more = st + 1 < nsteps;
    if (more) gload(st + 1);
    compute(cur);
    if (more) lstore(cur ^ 1);
    __syncthreads();
  }

  if (r > 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t mrow = imin(m0 + 128 * wm + 32 * i + l32, M - 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t kcol = imin(k0 + 128 * wn + 32 * j + l32, K - 1);
        f32x16 tmp;
#pragma unroll
        for (int v = 0; v < 16; ++v) tmp[v] = 0.f;
        for (int rs = 0; rs < rp / 16; ++rs) {
          const bf16x8 a = as_bf16x8(ld16(ul + mrow * rp + 16 * rs + 8 * h));
          uint32_t bv[4] = {0u, 0u, 0u, 0u};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int jj = 16 * rs + 8 * h + e;
            const uint32_t val = jj < r ? static_cast<uint32_t>(Al[static_cast<int64_t>(jj) * K + kcol]) : 0u;
            bv[e >> 1] |= val << (16 * (e & 1));
          }
          tmp = mfma32(a, as_bf16x8(u32x4{bv[0], bv[1], bv[2], bv[3]}), tmp);
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] += scale * tmp[v];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t kk = k0 + 128 * wn + 32 * j + l32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t mm = m0 + 128 * wm + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
        if (mm < M && kk < K) dx[mm * K + kk] = bf16_bits(acc[i][j][v]);
      }
    }
}

// ---------------------------------------------------------------------------
// dispatch: LoRA down-projection, then the small-M or the tiled kernel
// ---------------------------------------------------------------------------
hipError_t launch_lora_fwd(const uint16_t* x, int64_t M, int64_t N, int64_t K, const uint8_t* packed,
                           const int8_t* qscale, const float* step, const uint16_t* A, const uint16_t* B,
                           int r, float alpha, uint16_t* y, void* ws, const Codebook& cb,
                           hipStream_t stream) {
  const WsLayout L = ws_layout(0, M, N, K, r);
  char* wsb = static_cast<char*>(ws);
  const float scale = r > 0 ? alpha / static_cast<float>(r) : 0.0f;
  const int rp = r > 0 ? static_cast<int>(rank_pad(r)) : 0;
  void* lora = r > 0 ? static_cast<void*>(wsb + L.lora_off) : nullptr;
  if (r > 0) {
    const hipError_t e = launch_lora_down(true, x, M, K, A, r, lora, stream);
    if (e != hipSuccess) return e;
  }
  if (M <= kSmallM)
    return launch_fwd_small(x, M, N, K, packed, qscale, step, static_cast<const float*>(lora),
                            static_cast<int>(lora_splits(M, K)), rp, B, r, scale, y, cb, stream);
  const int64_t tiles = cdiv(M, kTile) * cdiv(N, kTile);
  hipLaunchKernelGGL(k_gemm_fwd, dim3(static_cast<unsigned>(tiles)), dim3(256), 0, stream, x, M, N, K, packed,
                     qscale, step, static_cast<const uint16_t*>(lora), rp, B, r, scale, y, cb);
  return hipGetLastError();
}

hipError_t launch_bwd_dx(const uint16_t* dy, int64_t M, int64_t N, int64_t K, const uint8_t* packed,
                         const int8_t* qscale, const float* step, const uint16_t* A, const uint16_t* B,
                         int r, float alpha, uint16_t* dx, void* ws, const Codebook& cb,
                         hipStream_t stream) {
  const WsLayout L = ws_layout(1, M, N, K, r);
  char* wsb = static_cast<char*>(ws);
  const float scale = r > 0 ? alpha / static_cast<float>(r) : 0.0f;
  const int rp = r > 0 ? static_cast<int>(rank_pad(r)) : 0;
  void* lora = r > 0 ? static_cast<void*>(wsb + L.lora_off) : nullptr;
  if (r > 0) {
    const hipError_t e = launch_lora_down(false, dy, M, N, B, r, lora, stream);
    if (e != hipSuccess) return e;
  }
  if (M <= kSmallM)
    return launch_bwd_small(dy, M, N, K, packed, qscale, step, static_cast<const float*>(lora),
                            static_cast<int>(lora_splits(M, N)), rp, A, r, scale,
                            reinterpret_cast<float*>(wsb + L.part_off), dx, cb, stream);
  const int64_t tiles = cdiv(M, kTile) * cdiv(K, kTile);
  hipLaunchKernelGGL(k_gemm_bwd, dim3(static_cast<unsigned>(tiles)), dim3(256), 0, stream, dy, M, N, K, packed,
                     qscale, step, static_cast<const uint16_t*>(lora), rp, A, r, scale, dx, cb);
  return hipGetLastError();
}

}  // namespace qnf4
