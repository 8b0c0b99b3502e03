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
//   k_gemm_fwd    M > 16: 256x256 output tile, 4 waves of 128x128, 64-deep
//                 K steps double-buffered in LDS; one thread per weight row
//                 dequantizes a whole 64-block into the LDS B tile; 32x32x16
//                 bf16 MFMA with fp32 accumulation; LoRA as a rank-r MFMA in
//                 the epilogue. MFMA-bound.
//   k_gemm_bwd    M > 16: same tiling over dX [M, K]; the contraction runs over
//                 W's rows, so the dequantized tile is stored row-major and
//                 read transposed with ds_read_b64_tr_b16.
//   k_bwd_small   M <= 16 backward: 64-column tiles, row slices reduced by
//   k_bwd_finish  a second kernel that also adds the LoRA term.
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

// ---------------------------------------------------------------------------
// k_lora_down: out[m][j] = sum_k in[m][k] * W(j, k),  j < rp (rows j >= r are 0)
//   WROW:  W(j,k) = W[j*Kc + k]  (A of the forward, [r][K])
//   !WROW: W(j,k) = W[k*r + j]   (B of the backward, [N][r])
// Grid (ceil(M/64), S): 4 waves of 16 rows; blockIdx.y takes a K-slice.
// PARTIAL: fp32 partial sums [S][M][rp]; else bf16 [M][rp] (S must be 1).
// ---------------------------------------------------------------------------
template <bool WROW, bool PARTIAL>
__global__ __launch_bounds__(256) void k_lora_down(const uint16_t* __restrict__ in, int64_t M, int64_t Kc,
                                                   const uint16_t* __restrict__ W, int r, int rp, int S,
                                                   void* __restrict__ out) {
  __shared__ u32x4 wl[128 * 8];              // [j][8 chunks] of one 64-deep K chunk
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * 64 + w * 16;
  const int s = blockIdx.y;
  const int64_t nch = cdiv(Kc, 64);           // the last chunk may be partial
  const int64_t c_beg = s * nch / S, c_end = (s + 1) * nch / S;
  const int ntile = rp / 16;
  const int64_t arow = imin(m0 + (lane & 15), M - 1);
  const uint16_t* in_row = in + arow * Kc;
  f32x4 acc[8];
#pragma unroll
  for (int jt = 0; jt < 8; ++jt) acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t c = c_beg; c < c_end; ++c) {
    const int64_t k0 = c * 64;
    if (WROW) {
      for (int q = t; q < rp * 8; q += 256) {
        const int j = q >> 3, ch = q & 7;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (j < r && k0 + ch * 8 < Kc) v = ld16(W + static_cast<int64_t>(j) * Kc + k0 + ch * 8);
        wl[j * 8 + (ch ^ (j & 7))] = v;
      }
    } else {
      uint16_t* wl16 = reinterpret_cast<uint16_t*>(wl);
      for (int q = t; q < rp * 64; q += 256) {
        const int kk = q / rp, j = q - kk * rp;
        const uint16_t v = (j < r && k0 + kk < Kc) ? W[(k0 + kk) * r + j] : static_cast<uint16_t>(0);
        wl16[(j * 8 + ((kk >> 3) ^ (j & 7))) * 8 + (kk & 7)] = v;
      }
    }
    __syncthreads();
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const int64_t ka = k0 + 32 * kh + 8 * (lane >> 4);   // Kc is a multiple of 8
      const bf16x8 a = as_bf16x8(ka < Kc ? ld16(in_row + ka) : u32x4{0u, 0u, 0u, 0u});
#pragma unroll
      for (int jt = 0; jt < 8; ++jt) {
        if (jt < ntile) {
          const int j = 16 * jt + (lane & 15);
          const bf16x8 b = as_bf16x8(wl[j * 8 + ((4 * kh + (lane >> 4)) ^ (j & 7))]);
          acc[jt] = mfma16(a, b, acc[jt]);
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int jt = 0; jt < 8; ++jt) {
    if (jt >= ntile) break;
    const int j = 16 * jt + (lane & 15);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t m = m0 + 4 * (lane >> 4) + v;
      if (m < M) {
        if (PARTIAL)
          static_cast<float*>(out)[(s * M + m) * rp + j] = acc[jt][v];
        else
          static_cast<uint16_t*>(out)[m * rp + j] = bf16_bits(acc[jt][v]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// k_gemv_fwd (M <= 16). Workgroup = 16 weight rows x all of K, 8 waves.
// Lane l: g = l/16 picks one of the 4 blocks of a 256-deep super-step, c = l%16
// is both the weight row (B operand column) and the x row (A operand row).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(512) void k_gemv_fwd(const uint16_t* __restrict__ x, int64_t M, int64_t N,
                                                  int64_t K, const uint8_t* __restrict__ packed,
                                                  const int8_t* __restrict__ qscale,
                                                  const float* __restrict__ step,
                                                  const float* __restrict__ tpart, int St, int rp,
                                                  const uint16_t* __restrict__ Bl, int r, float scale,
                                                  uint16_t* __restrict__ y, Codebook cb) {
  __shared__ f32x4 red[8][64];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int64_t n = imin(n0 + c, N - 1);
  const int64_t m = imin(static_cast<int64_t>(c), M - 1);
  const int64_t nbr = K / 64;
  const int64_t nss = cdiv(nbr, 4);
  const uint8_t* prow = packed + n * (K / 2);
  const uint16_t* xrow = x + m * K;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int64_t ss = w; ss < nss; ss += 8) {
    const int64_t kb = ss * 4 + g;
    const bool valid = kb < nbr;
    const int64_t kbc = valid ? kb : nbr - 1;
    const u32x4 p0 = ld16(prow + kbc * 32);
    const u32x4 p1 = ld16(prow + kbc * 32 + 16);
    const int64_t blk = n * nbr + kbc;
    const float sc = valid ? block_scale(qscale[blk], step[blk >> 8]) : 0.0f;
    const uint16_t* xk = xrow + kbc * 64;
    u32x4 xa[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) xa[j] = ld16(xk + 8 * j);
    const MagTable tb = make_table(cb, sc);
    const uint32_t pw[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = mfma16(as_bf16x8(xa[j]), as_bf16x8(decode8(pw[j], tb)), acc);
  }
  red[w][lane] = acc;
  __syncthreads();
  if (w != 0) return;
  acc = red[0][lane];
#pragma unroll
  for (int i = 1; i < 8; ++i) acc += red[i][lane];

  if (r > 0) {
    f32x4 tmp = {0.f, 0.f, 0.f, 0.f};
    const uint16_t* brow = Bl + n * r;
    for (int js = 0; js < rp / 32; ++js) {
      const int j0 = 32 * js + 8 * g;
      float tv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) tv[e] = 0.f;
      for (int s = 0; s < St; ++s) {
        const float* tp = tpart + (s * M + m) * rp + j0;
        const f32x4 u0 = *reinterpret_cast<const f32x4*>(tp);
        const f32x4 u1 = *reinterpret_cast<const f32x4*>(tp + 4);
        tv[0] += u0.x; tv[1] += u0.y; tv[2] += u0.z; tv[3] += u0.w;
        tv[4] += u1.x; tv[5] += u1.y; tv[6] += u1.z; tv[7] += u1.w;
      }
      const u32x4 a = {pack_bf16x2(tv[0], tv[1]), pack_bf16x2(tv[2], tv[3]), pack_bf16x2(tv[4], tv[5]),
                       pack_bf16x2(tv[6], tv[7])};
      const u32x4 b = load_row8(brow, j0, r, (r & 7) == 0);
      tmp = mfma16(as_bf16x8(a), as_bf16x8(b), tmp);
    }
    acc += scale * tmp;
  }
  const int64_t nn = n0 + c;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t mm = 4 * g + v;
    if (mm < M && nn < N) y[mm * N + nn] = bf16_bits(acc[v]);
  }
}

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

__global__ __launch_bounds__(256, 1) void k_gemm_fwd(const uint16_t* __restrict__ x, int64_t M, int64_t N,
                                                     int64_t K, const uint8_t* __restrict__ packed,
                                                     const int8_t* __restrict__ qscale,
                                                     const float* __restrict__ step,
                                                     const uint16_t* __restrict__ tl, int rp,
                                                     const uint16_t* __restrict__ Bl, int r, float scale,
                                                     uint16_t* __restrict__ y, Codebook cb) {
  __shared__ u32x4 smem[4 * kChunks];        // A[2], B[2]: 128 KB
  u32x4* As = smem;
  u32x4* Bs = smem + 2 * kChunks;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int h = lane >> 5, l32 = lane & 31;
  const int ntm = static_cast<int>(cdiv(M, kTile)), ntn = static_cast<int>(cdiv(N, kTile));
  int tm, tn;
  tile_of(blockIdx.x, ntm, ntn, tm, tn);
  const int64_t m0 = static_cast<int64_t>(tm) * kTile, n0 = static_cast<int64_t>(tn) * kTile;
  const int64_t nbr = K / 64;

  // global -> register staging assignments
  const int ach = t & 7, arow0 = t >> 3;
  const uint16_t* aptr[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) aptr[i] = x + imin(m0 + arow0 + 32 * i, M - 1) * K + ach * 8;
  const int64_t brow = imin(n0 + t, N - 1);
  const uint8_t* bptr = packed + brow * (K / 2);
  const int64_t bblk = brow * nbr;

  u32x4 areg[8];
  u32x4 b0, b1;
  int8_t qv;
  float dv;
  auto gload = [&](int64_t kt) {
#pragma unroll
    for (int i = 0; i < 8; ++i) areg[i] = ld16(aptr[i] + kt * 64);
    b0 = ld16(bptr + kt * 32);
    b1 = ld16(bptr + kt * 32 + 16);
    qv = qscale[bblk + kt];
    dv = step[(bblk + kt) >> 8];
  };
  auto lstore = [&](int buf) {
    u32x4* Ab = As + buf * kChunks;
    u32x4* Bb = Bs + buf * kChunks;
#pragma unroll
    for (int i = 0; i < 8; ++i) Ab[a_slot(arow0 + 32 * i, ach)] = areg[i];
    const MagTable tb = make_table(cb, block_scale(qv, dv));
    const uint32_t pw[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) Bb[a_slot(t, ch)] = decode8(pw[ch], tb);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

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
      for (int j = 0; j < 4; ++j) bfr[j] = as_bf16x8(Bb[(128 * wn + 32 * j + l32) * 8 + sw]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
  };

  gload(0);
  lstore(0);
  __syncthreads();
  for (int64_t kt = 0; kt < nbr; ++kt) {
    const int cur = static_cast<int>(kt & 1);
    const bool more = kt + 1 < nbr;
    if (more) gload(kt + 1);
    compute(cur);
    if (more) lstore(cur ^ 1);
    __syncthreads();
  }

  if (r > 0) {
    const bool vec_ok = (r & 7) == 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t mrow = imin(m0 + 128 * wm + 32 * i + l32, M - 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t nrow = imin(n0 + 128 * wn + 32 * j + l32, N - 1);
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
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t nn = n0 + 128 * wn + 32 * j + l32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t mm = m0 + 128 * wm + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
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

__device__ __forceinline__ s16x4 ds_read_tr(const u32x4* base, int elem_off) {
  // generic -> LDS address space (the pointer always refers to __shared__ memory)
  lds_short* p = (lds_short*)(const_cast<short*>(reinterpret_cast<const short*>(base))) + elem_off;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
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
// Small-M backward: grid (K/64 column tiles, S row slices). 256 weight rows per
// step are dequantized (one 64-block each) into LDS; 4 waves each contract 64
// of them with 16x16x32 MFMAs (B read transposed). fp32 partials [S][M][K].
// ---------------------------------------------------------------------------
__device__ __forceinline__ int sm_slot(int row, int ch) {
  const int g = ((row & 3) << 1) | ((row >> 2) & 1);
  return row * 8 + (ch ^ g);
}

__global__ __launch_bounds__(256) void k_bwd_small(const uint16_t* __restrict__ dy, int64_t M, int64_t N,
                                                   int64_t K, const uint8_t* __restrict__ packed,
                                                   const int8_t* __restrict__ qscale,
                                                   const float* __restrict__ step, int S,
                                                   float* __restrict__ part, Codebook cb) {
  __shared__ u32x4 Bs[256 * 8];
  __shared__ f32x4 red[4][4][64];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int64_t kt = blockIdx.x;             // 64-column tile == block column kt
  const int s = blockIdx.y;
  const int64_t nbr = K / 64;
  const int64_t nsteps = cdiv(N, 256);
  const int64_t st_beg = s * nsteps / S, st_end = (s + 1) * nsteps / S;
  const int64_t m = imin(static_cast<int64_t>(lane & 15), M - 1);
  const int G = lane >> 4, j16 = lane & 15;
  f32x4 acc[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t st = st_beg; st < st_end; ++st) {
    {
      const int64_t row = imin(st * 256 + t, N - 1);
      const uint8_t* p = packed + row * (K / 2) + kt * 32;
      const u32x4 b0 = ld16(p), b1 = ld16(p + 16);
      const int64_t blk = row * nbr + kt;
      const MagTable tb = make_table(cb, block_scale(qscale[blk], step[blk >> 8]));
      const uint32_t pw[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
      for (int ch = 0; ch < 8; ++ch) Bs[sm_slot(t, ch)] = decode8(pw[ch], tb);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int64_t ncol = st * 256 + 64 * w + 32 * ks + 8 * G;
      const u32x4 av = ncol < N ? ld16(dy + m * N + ncol) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int cbk = 0; cbk < 4; ++cbk) {
        const int col = 16 * cbk + 4 * (j16 & 3);
        s16x4 v[2];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int row = 64 * w + 32 * ks + 8 * G + 4 * q + (j16 >> 2);
          v[q] = ds_read_tr(Bs, sm_slot(row, col >> 3) * 8 + (col & 4));
        }
        const bf16x8 b = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7));
        acc[cbk] = mfma16(as_bf16x8(av), b, acc[cbk]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int cbk = 0; cbk < 4; ++cbk) red[w][cbk][lane] = acc[cbk];
  __syncthreads();
  {
    const int cbk = t >> 6, ln = t & 63;
    f32x4 sum = red[0][cbk][ln];
#pragma unroll
    for (int i = 1; i < 4; ++i) sum += red[i][cbk][ln];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t mm = 4 * (ln >> 4) + v;
      if (mm < M) part[(s * M + mm) * K + kt * 64 + 16 * cbk + (ln & 15)] = sum[v];
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
  if (r > 0) {
    if (t < rp) {
      float u = 0.f;
      for (int s = 0; s < Su; ++s) u += upart[(s * M + m) * rp + t];
      us[t] = bf16_lo(static_cast<uint32_t>(bf16_bits(u)));
    }
    __syncthreads();
  }
  if (k >= K) return;
  float v = 0.f;
  for (int s = 0; s < S; ++s) v += part[(s * M + m) * K + k];
  if (r > 0) {
    float l = 0.f;
    for (int j = 0; j < r; ++j) l += us[j] * bf16_lo(static_cast<uint32_t>(Al[static_cast<int64_t>(j) * K + k]));
    v += scale * l;
  }
  dx[m * K + k] = bf16_bits(v);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_lora_fwd(const uint16_t* x, int64_t M, int64_t N, int64_t K, const uint8_t* packed,
                           const int8_t* qscale, const float* step, const uint16_t* A, const uint16_t* B,
                           int r, float alpha, uint16_t* y, void* ws, const Codebook& cb,
                           hipStream_t stream) {
  const WsLayout L = ws_layout(0, M, N, K, r);
  char* wsb = static_cast<char*>(ws);
  const float scale = r > 0 ? alpha / static_cast<float>(r) : 0.0f;
  const int rp = r > 0 ? static_cast<int>(rank_pad(r)) : 0;
  if (M <= kSmallM) {
    const int St = static_cast<int>(lora_splits(M, K));
    float* tpart = r > 0 ? reinterpret_cast<float*>(wsb + L.lora_off) : nullptr;
    if (r > 0)
      hipLaunchKernelGGL((k_lora_down<true, true>), dim3(static_cast<unsigned>(cdiv(M, 64)), St), dim3(256), 0,
                         stream, x, M, K, A, r, rp, St, static_cast<void*>(tpart));
    hipLaunchKernelGGL(k_gemv_fwd, dim3(static_cast<unsigned>(cdiv(N, 16))), dim3(512), 0, stream, x, M, N, K,
                       packed, qscale, step, tpart, St, rp, B, r, scale, y, cb);
  } else {
    uint16_t* tl = r > 0 ? reinterpret_cast<uint16_t*>(wsb + L.lora_off) : nullptr;
    if (r > 0)
      hipLaunchKernelGGL((k_lora_down<true, false>), dim3(static_cast<unsigned>(cdiv(M, 64)), 1), dim3(256), 0,
                         stream, x, M, K, A, r, rp, 1, static_cast<void*>(tl));
    const int64_t tiles = cdiv(M, kTile) * cdiv(N, kTile);
    hipLaunchKernelGGL(k_gemm_fwd, dim3(static_cast<unsigned>(tiles)), dim3(256), 0, stream, x, M, N, K, packed,
                       qscale, step, tl, rp, B, r, scale, y, cb);
  }
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
  if (M <= kSmallM) {
    const int Su = static_cast<int>(lora_splits(M, N));
    float* upart = r > 0 ? reinterpret_cast<float*>(wsb + L.lora_off) : nullptr;
    if (r > 0)
      hipLaunchKernelGGL((k_lora_down<false, true>), dim3(static_cast<unsigned>(cdiv(M, 64)), Su), dim3(256), 0,
                         stream, dy, M, N, B, r, rp, Su, static_cast<void*>(upart));
    const int Sb = static_cast<int>(bwd_small_splits(N, K));
    float* part = reinterpret_cast<float*>(wsb + L.part_off);
    hipLaunchKernelGGL(k_bwd_small, dim3(static_cast<unsigned>(K / 64), Sb), dim3(256), 0, stream, dy, M, N, K,
                       packed, qscale, step, Sb, part, cb);
    hipLaunchKernelGGL(k_bwd_finish, dim3(static_cast<unsigned>(cdiv(K, 256)), static_cast<unsigned>(M)),
                       dim3(256), 0, stream, part, Sb, M, K, upart, Su, rp, A, r, scale, dx);
  } else {
    uint16_t* ul = r > 0 ? reinterpret_cast<uint16_t*>(wsb + L.lora_off) : nullptr;
    if (r > 0)
      hipLaunchKernelGGL((k_lora_down<false, false>), dim3(static_cast<unsigned>(cdiv(M, 64)), 1), dim3(256), 0,
                         stream, dy, M, N, B, r, rp, 1, static_cast<void*>(ul));
    const int64_t tiles = cdiv(M, kTile) * cdiv(K, kTile);
    hipLaunchKernelGGL(k_gemm_bwd, dim3(static_cast<unsigned>(tiles)), dim3(256), 0, stream, dy, M, N, K, packed,
                       qscale, step, ul, rp, A, r, scale, dx, cb);
  }
  return hipGetLastError();
}

}  // namespace qnf4
