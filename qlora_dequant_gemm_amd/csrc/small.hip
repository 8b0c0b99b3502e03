// Decode-shaped (M <= 16) fused NF4-dequant backward for gfx950, over a table
// of weights in one launch.
//
//   dX_p = bf16( dY_p . W_p' + (alpha/r) . u_p . A_p ),  u_p = dY_p . B_p
//
// for every weight p of the table ("A 65B fine-tune on the GPU you already
// have", figure 2: the gradient flows through the frozen weights, which become
// bf16 block by block right before the multiply; "QLoRA" (techbytebybyte),
// "Follow one QLoRA training step"). At these shapes each weight is used by at
// most 16 rows, so the kernels stream the 0.516 bytes/param stored weight once
// and are bound by that stream, by its latency and by the VALU work of
// decoding it.
//
// The contraction runs over W's rows while a packed code word holds 8
// consecutive columns of one row (all with one block scale), so each wave
// decodes its codes with the blocks' tables into a bf16 tile of its own in LDS
// and reads the MFMA B operands (several rows of one column) back transposed
// (ds_read_b64_tr_b16), against dY. A wave's LDS operations complete in order,
// so its tile needs no barrier.
//
// Work items are a column range of dX x a range of W's rows, one workgroup of
// four waves each. Rows are split into S ranges when a launch has too few
// column ranges to fill the chip, or to bound the items; every split writes
// fp32 partial sums and the last split of a column range to arrive (an arrival
// counter in the workspace) adds them in split order, so results do not depend
// on scheduling. Items of one column range run on one XCD (consecutive
// workgroup ids go round robin over the 8 XCDs), so their partials stay in
// that XCD's L2. Two item shapes:
//   narrow  64 columns (one block column); the waves take 64-row sub-tiles in
//           turn, lane (g, c) decoding row 16g + c. The partials of a split
//           are small (64 x M fp32), so a single call on one weight, whose rows
//           must be split many ways to fill the chip, finishes soon.
//   wide    256 columns (four blocks); wave w takes rows 64w .. 64w + 63 of
//           each 256-row super-step, lane (g, c) decoding block g of rows
//           16ch + c (one load covers 16 rows x 64 contiguous bytes), four
//           chunks of codes one super-step ahead, with dY (and for rank 16 the
//           B rows) staged in LDS once for the four waves. Streams a launch
//           with many column ranges (a batch of weights) at the higher rate.
//
// LoRA. The B rows go through the same transposed path, so each item also
// accumulates u_s = dY . B over its own rows. After the main loop the four
// waves' parts of the partial sums and of u_s are added through LDS (fixed
// order), and (alpha/r) . u_s . A over the item's columns is added with
// (alpha/r) . u_s carried as the sum of two bf16 values (hi + lo, about 16
// significant bits), so splitting the rows leaves the LoRA term exact to
// fp32-level rounding instead of requiring the full u before any output.
//
// Decode order. decode8_perm yields the 8 weights of a code dword in the order
// 0 2 4 6 1 3 5 7; the tiles' columns keep that order (the A rows of the LoRA
// term are permuted the same way), and the outputs go to their true columns.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "mm_common.hpp"

namespace qnf4 {

constexpr int kDbWaves = 4;
constexpr int kDbBufWord3 = 0x00020000;        // raw buffer descriptor word 3 on gfx9-family parts
// A wave-uniform value moved to a scalar register: buffer descriptors built
// from it stay scalar (a descriptor the compiler holds in vector registers
// turns every load through it into a per-lane loop).
__device__ __forceinline__ int sgpr(int v) { return __builtin_amdgcn_readfirstlane(v); }
constexpr int kDnCols = 64;                    // narrow items: dX columns (one block column)
constexpr int kDnSub = 64;                     //   weight rows per sub-tile
constexpr int kDnUChunks = 192;                //   16-byte chunks of one rank tile's B rows (padded)
constexpr int kDwCols = 256;                   // wide items: dX columns
constexpr int kDwSS = 256;                     //   weight rows per super-step

// position p of a decoded 8-group holds element pi(p) (order 0 2 4 6 1 3 5 7)
__device__ __forceinline__ int db_col(int p) { return (p & ~7) | ((p & 3) << 1) | ((p >> 2) & 1); }

__device__ __forceinline__ f32x4 mfma16k16(const s16x4& a, const s16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int db_item_of(int wg, int grid) {
  // grid is a multiple of 8: XCD (wg % 8) gets items [xcd * grid/8, ...)
  return (wg & 7) * (grid >> 3) + (wg >> 3);
}

// ===========================================================================
// Narrow items: one 64-column block column x a range of 64-row sub-tiles.
// ===========================================================================
// 16-byte chunk ch (0..7) of row `row` (0..63) of the 64 x 64 bf16 tile. The
// writes (16 lanes: 16 consecutive rows, one chunk) and the transposed reads
// (32 lanes: 8 rows, two adjacent chunks) each touch all 64 banks once.
__device__ __forceinline__ int dn_slot(int row, int ch) {
  const int i = (row >> 1) & 7;
  return row * 8 + (ch ^ (((i & 1) << 1) | ((i >> 1) & 1) | (i & 4)));
}
// chunk ch (0, 1) of row `row` of the B rows of one rank tile (16 ranks); a
// chunk of padding after every 8 rows keeps the transposed reads conflict-free
__device__ __forceinline__ int dn_uslot(int row, int ch) { return row * 2 + ch + 8 * (row >> 3); }

// B operand of a 16x16x32 MFMA (rows row0 .. row0 + 7 of a tile, column
// col0 + c) from the decoded tile (kU = false) or the B rows of a rank tile
// (kU = true): two transposed 8-byte reads, rows row0 + 4q + c/4, columns
// col0 + 4 (c % 4) .. + 3
template <bool kU>
__device__ __forceinline__ bf16x8 dn_operand(const u32x4* base, int row0, int col0, int c) {
  s16x4 v[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int row = row0 + 4 * q + (c >> 2), col = col0 + 4 * (c & 3);
    const int sl = kU ? dn_uslot(row, col >> 3) : dn_slot(row, col >> 3);
    v[q] = ds_read_tr(base, sl * 8 + (col & 4));
  }
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// NTU: rank tiles of 16 (0: no adapter; else a power of two with 16 NTU >= r).
template <int NTU>
__global__ __launch_bounds__(64 * kDbWaves, 3) void k_dec_bwd_narrow(DecBwdBatch bt, Codebook cb) {
  constexpr int kU = NTU > 0 ? NTU : 1;
  // per wave: the decoded sub-tile (8 KB; then its accumulators for the
  // cross-wave sums, then the A rows of its LoRA term) and the B rows of a
  // sub-tile (then its part of u_s, then u_s)
  __shared__ u32x4 T0[512], T1[512], T2[512], T3[512];
  __shared__ u32x4 U0[kDnUChunks * kU], U1[kDnUChunks * kU], U2[kDnUChunks * kU], U3[kDnUChunks * kU];
  __shared__ int last_flag;

  const int item = db_item_of(blockIdx.x, gridDim.x);
  if (item >= bt.items) return;
  int pi = 0;
#pragma unroll
  for (int i = 1; i < kDecMaxProblems; ++i)
    if (i < bt.count && item >= bt.p[i].item0) pi = i;
  const DecBwdProblem& P = bt.p[pi];

  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int g = lane >> 4, c = lane & 15;
  u32x4* const Tw = w == 0 ? T0 : w == 1 ? T1 : w == 2 ? T2 : T3;
  u32x4* const Uw = w == 0 ? U0 : w == 1 ? U1 : w == 2 ? U2 : U3;
  const int M = bt.M, r = bt.r;
  const int N = P.N, K = P.K;                  // sizes fit 32 bits (N, K <= 2^21)
  const int nbr = K / 64;
  const int local = item - P.item0;
  const int kb = local / P.S, s = local - (local / P.S) * P.S;    // block column, row split
  const int nst = (N + kDnSub - 1) / kDnSub;
  const int st0 = s * P.sps;
  const int st1 = st0 + P.sps < nst ? st0 + P.sps : nst;
  const int row = 16 * g + c;                  // this lane's row of a sub-tile

  const uint32_t coff = static_cast<uint32_t>(row * (K / 2) + kb * 32);
  const uint32_t qoff = static_cast<uint32_t>(row * nbr + kb);
  const int64_t ngroups = (static_cast<int64_t>(N) * nbr + 255) >> 8;
  const __amdgpu_buffer_rsrc_t dyrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(P.dy), 0, M * N * 2, kDbBufWord3);
  const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(NTU > 0 ? P.B : P.dy), 0, NTU > 0 ? N * r * 2 : 0, kDbBufWord3);

  // the A rows of this wave's LoRA columns (16 w .. 16 w + 15 of the tile),
  // loaded now and used after the main loop: lane l < 32 holds chunk 2w + l % 2
  // of A row 16 jt + l / 2
  u32x4 apre[kU];
  if constexpr (NTU > 0) {
    const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(P.A), 0, r * K * 2, kDbBufWord3);
#pragma unroll
    for (int jt = 0; jt < NTU; ++jt) {
      const int j = 16 * jt + (lane >> 1);
      const uint32_t ao = (lane < 32 && j < r)
                              ? static_cast<uint32_t>((j * K + kb * 64 + 8 * (2 * w + (lane & 1))) * 2)
                              : 0x80000000u;
      apre[jt] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ars, ao, 0, 0));
    }
  }

  struct Stage {
    u32x4 cw0, cw1;       // the 32 code bytes of block kb of row n0 + row
    uint32_t q;           // its scale code (byte)
    float d;              // its second-level step
    u32x4 dyf[2];         // dY[c][n0 + 32 ks + 8g .. + 7], ks = 0, 1
    u32x4 bu[kU][2];      // B[n0 + row][16 jt .. 16 jt + 15]
  };
  // Operands of sub-tile st. The row-dependent parts sit in the descriptors'
  // base addresses (scalar), so most lane offsets stay fixed; rows past N
  // read as zero codes with a zero scale code, i.e. zero weights.
  auto issue = [&](int st, Stage& S) {
    const int n0 = st * kDnSub;
    const int rows = N - n0 < kDnSub ? N - n0 : kDnSub;
    const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(P.packed + static_cast<int64_t>(n0) * (K / 2)), 0, rows * (K / 2), kDbBufWord3);
    S.cw0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(crs, coff, 0, 0));
    S.cw1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(crs, coff + 16, 0, 0));
    const int64_t sb = static_cast<int64_t>(n0) * nbr;      // first block of the sub-tile
    const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(P.qscale + sb), 0, rows * nbr, kDbBufWord3);
    S.q = __builtin_amdgcn_raw_buffer_load_b8(qrs, qoff, 0, 0);
    const int64_t g0 = sb >> 8;
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(P.step + g0), 0, static_cast<int>((ngroups - g0) * 4), kDbBufWord3);
    S.d = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                        srs, static_cast<uint32_t>((((sb & 255) + qoff) >> 8) * 4), 0, 0));
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int n = n0 + 32 * ks + 8 * g;      // N is a multiple of 8: a group is in or out
      const uint32_t o = n < N ? static_cast<uint32_t>((c * N + n) * 2) : 0x80000000u;
      S.dyf[ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(dyrs, o, 0, 0));
    }
    if constexpr (NTU > 0) {
#pragma unroll
      for (int jt = 0; jt < NTU; ++jt) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int j = 16 * jt + 8 * h;
          const uint32_t bo = static_cast<uint32_t>(((n0 + row) * r + j) * 2);
          if ((r & 7) == 0) {
            S.bu[jt][h] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(brs, j < r ? bo : 0x80000000u, 0, 0));
          } else {                              // rows of B not 16-byte aligned: one rank at a time
            uint32_t e16[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
              e16[e] = __builtin_amdgcn_raw_buffer_load_b16(brs, j + e < r ? bo + 2 * e : 0x80000000u, 0, 0);
            S.bu[jt][h] = u32x4{e16[0] | (e16[1] << 16), e16[2] | (e16[3] << 16), e16[4] | (e16[5] << 16),
                                e16[6] | (e16[7] << 16)};
          }
        }
      }
    }
  };

  f32x4 acc[4], uacc[kU];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int jt = 0; jt < kU; ++jt) uacc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto consume = [&](const Stage& S) {
    const float sc = block_scale(static_cast<int8_t>(S.q), S.d);
    const MagTable tb = make_table(cb, sc);
    const uint32_t pw[8] = {S.cw0.x, S.cw0.y, S.cw0.z, S.cw0.w, S.cw1.x, S.cw1.y, S.cw1.z, S.cw1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) Tw[dn_slot(row, j)] = decode8_perm(pw[j], tb);
    if constexpr (NTU > 0) {
#pragma unroll
      for (int jt = 0; jt < NTU; ++jt)
#pragma unroll
        for (int h = 0; h < 2; ++h) Uw[kDnUChunks * jt + dn_uslot(row, h)] = S.bu[jt][h];
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 a = as_bf16x8(S.dyf[ks]);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, dn_operand<false>(Tw, 32 * ks + 8 * g, 16 * ct, c),
                                                          acc[ct], 0, 0, 0);
      if constexpr (NTU > 0) {
#pragma unroll
        for (int jt = 0; jt < NTU; ++jt)
          uacc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              a, dn_operand<true>(Uw + kDnUChunks * jt, 32 * ks + 8 * g, 0, c), uacc[jt], 0, 0, 0);
      }
    }
  };

  // this wave's sub-tiles: st0 + w, st0 + w + 4, ...
  const int nw = st1 - st0 - w > 0 ? (st1 - st0 - w + kDbWaves - 1) / kDbWaves : 0;
  Stage s0, s1;
  int i = 0;
  if (nw > 0) issue(st0 + w, s0);
  for (; i + 1 < nw; i += 2) {
    issue(st0 + w + kDbWaves * (i + 1), s1);
    consume(s0);
    if (i + 2 < nw) issue(st0 + w + kDbWaves * (i + 2), s0);
    consume(s1);
  }
  if (i < nw) consume(s0);

  // ---- the four waves' parts, summed in wave order; wave w keeps tile w ----
  __syncthreads();
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) Tw[ct * 64 + lane] = __builtin_bit_cast(u32x4, acc[ct]);
  if constexpr (NTU > 0) {
#pragma unroll
    for (int jt = 0; jt < NTU; ++jt) Uw[jt * 64 + lane] = __builtin_bit_cast(u32x4, uacc[jt]);
  }
  __syncthreads();
  const int idx = w * 64 + lane;
  f32x4 fin = __builtin_bit_cast(f32x4, T0[idx]);
  fin += __builtin_bit_cast(f32x4, T1[idx]);
  fin += __builtin_bit_cast(f32x4, T2[idx]);
  fin += __builtin_bit_cast(f32x4, T3[idx]);
  f32x4 usum[kU];
  if constexpr (NTU > 0) {
    // u_s, lane (g, c) of rank tile jt holding u[4 g + v][16 jt + c]
#pragma unroll
    for (int jt = 0; jt < NTU; ++jt) {
      const int ui = jt * 64 + lane;
      usum[jt] = __builtin_bit_cast(f32x4, U0[ui]);
      usum[jt] += __builtin_bit_cast(f32x4, U1[ui]);
      usum[jt] += __builtin_bit_cast(f32x4, U2[ui]);
      usum[jt] += __builtin_bit_cast(f32x4, U3[ui]);
    }
  }
  __syncthreads();                               // every wave's reads of the exchange are done

  if constexpr (NTU > 0) {
    // (alpha/r) u_s as hi + lo bf16, the A operand of a 16x16x16 MFMA over
    // the ranks (lane (g, c): row m = c, ranks 16 jt + 4g .. + 3), through
    // this wave's own LDS
    float* const ush = reinterpret_cast<float*>(Uw);          // [16][16 kU]
#pragma unroll
    for (int jt = 0; jt < NTU; ++jt)
#pragma unroll
      for (int v = 0; v < 4; ++v) ush[(4 * g + v) * (16 * kU) + 16 * jt + c] = usum[jt][v];
    // the A rows of tile w's columns, in the tile's column order: rows
    // 0 .. 15 of this wave's tile memory, chunks 2w and 2w + 1
#pragma unroll
    for (int jt = 0; jt < NTU; ++jt) {
      if (lane < 32) Tw[dn_slot(lane >> 1, 2 * w + (lane & 1))] = perm8(apre[jt]);
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = bt.scale * ush[c * (16 * kU) + 16 * jt + 4 * g + e];
      const uint32_t h0 = pack_bf16x2(v[0], v[1]), h1 = pack_bf16x2(v[2], v[3]);
      const uint32_t l0 = pack_bf16x2(v[0] - bf16_lo(h0), v[1] - bf16_hi(h0));
      const uint32_t l1 = pack_bf16x2(v[2] - bf16_lo(h1), v[3] - bf16_hi(h1));
      // B operand: ranks 4g .. 4g + 3 (rows of the staged A) of column 16 w + c
      const int rr = 4 * g + (c >> 2), col = 16 * w + 4 * (c & 3);
      const s16x4 b = ds_read_tr(Tw, dn_slot(rr, col >> 3) * 8 + (col & 4));
      fin = mfma16k16(__builtin_bit_cast(s16x4, u32x2{h0, h1}), b, fin);
      fin = mfma16k16(__builtin_bit_cast(s16x4, u32x2{l0, l1}), b, fin);
    }
  }

  // lane (g, c) of tile w holds dX[4 g + v][64 kb + db_col(16 w + c)]
  const int kout = kb * 64 + db_col(16 * w + c);
  if (P.S == 1) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * g + v;
      if (m < M) P.dx[static_cast<int64_t>(m) * K + kout] = bf16_bits(fin[v]);
    }
    return;
  }
  // split N: partial sums [64 positions][Mp] of this split, then the last
  // split of the block column to arrive adds all of them in split order
  // (device-scope coherent stores and loads, the arrival counter as in the
  // decode-shaped forward)
  const int Mp = (M + 3) & ~3;
  float* const part_kb = bt.part + (P.part0 + static_cast<int64_t>(kb) * P.S) * (kDnCols * Mp);
  const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
      part_kb, 0, P.S * kDnCols * Mp * 4, kDbBufWord3);
  if (4 * g < M) {
    const uint32_t off = static_cast<uint32_t>(((s * kDnCols + 16 * w + c) * Mp + 4 * g) * 4);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, fin), prs, off, 0, 16);
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);                  // this wave's stores have completed
  __syncthreads();
  if (t == 0) {
    const unsigned old = __hip_atomic_fetch_add(bt.cnt + P.cnt0 + kb, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    last_flag = old == static_cast<unsigned>(P.S - 1);
  }
  __syncthreads();
  if (!last_flag) return;
  // thread t adds 4 consecutive values (position p, rows m0 .. m0 + 3) over
  // the splits, eight splits' loads in flight at a time
  if (t < kDnCols * Mp / 4) {
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
    for (int sp0 = 0; sp0 < P.S; sp0 += 8) {
      f32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t off = static_cast<uint32_t>(((sp0 + u) * kDnCols * Mp + 4 * t) * 4);
        v[u] = sp0 + u < P.S ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(prs, off, 0, 16))
                             : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) sum += v[u];
    }
    const int p = 4 * t / Mp, m0 = 4 * t - p * Mp;
    const int k = kb * 64 + db_col(p);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (m0 + e < M) P.dx[static_cast<int64_t>(m0 + e) * K + k] = bf16_bits(sum[e]);
  }
  if (t == 0) __hip_atomic_store(bt.cnt + P.cnt0 + kb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ===========================================================================
// Wide items: 256 columns x at most kDwMaxSps super-steps of 256 rows.
// ===========================================================================
// 16-byte chunk q (0..31) of row `row` (0..15) of a wave's 16 x 256 bf16
// tile. The writes (16 lanes: rows 0..15, one chunk) and the transposed reads
// (32 lanes: rows 0..7 or 8..15, two adjacent chunks) each touch all 64 banks
// once.
__device__ __forceinline__ int dw_slot(int row, int q) {
  return row * 32 + (q ^ (((row << 1) & 15) | (row >> 3)));
}
// chunk q of row m of the staged dY [16][256]: the 16 rows of a read phase
// (one logical chunk) land on 16 distinct bank groups
__device__ __forceinline__ int dw_yslot(int m, int q) { return m * 32 + (q ^ m); }

// NTU: rank tiles of 16 (0: no adapter; else a power of two with 16 NTU >= r).
// kSB: r == 16, the B rows of a super-step are staged in LDS with dY (else each
// wave loads the B rows of its chunks). kQuad: every K of the launch is a
// multiple of 256.
template <int NTU, bool kSB, bool kQuad>
__global__ __launch_bounds__(64 * kDbWaves, 2) void k_dec_bwd_wide(DecBwdBatch bt, Codebook cb) {
  constexpr int kU = NTU > 0 ? NTU : 1;
  static_assert(!kSB || NTU == 1, "staged B rows are one rank tile");
  // per wave: its decoded chunk (8 KB); after the main loop the same memory
  // holds the parts of u_s and of the partial sums for the cross-wave sums,
  // then the A rows of the LoRA term
  __shared__ u32x4 T0[512], T1[512], T2[512], T3[512];
  // dY over a super-step's rows, two super-steps; B rows likewise (r == 16)
  __shared__ u32x4 Y0[512], Y1[512];
  __shared__ u32x4 BS0[kSB ? 512 : 1], BS1[kSB ? 512 : 1];
  // per wave: the B rows of one chunk (16 rows x 16 kU ranks) when r != 16
  __shared__ u32x2 UB[kDbWaves][kSB || NTU == 0 ? 1 : 64 * kU];
  // scale code dword (the four blocks of the item) and step of every row of
  // the item
  __shared__ uint32_t lq[kQuad ? kDwSS * kDwMaxSps : 1];
  __shared__ float ld[kQuad ? kDwSS * kDwMaxSps : 1];
  __shared__ float Ush[16 * 16 * kU];
  __shared__ int last_flag;
  // workgroup barrier that orders the compiler's accesses to the shared
  // staging buffers too
  auto sync = [&] { lds_barrier_on(Y0, Y1, BS0, BS1, lq, ld); };

  const int item = db_item_of(blockIdx.x, gridDim.x);
  if (item >= bt.items) return;
  int pi = 0;
#pragma unroll
  for (int i = 1; i < kDecMaxProblems; ++i)
    if (i < bt.count && item >= bt.p[i].item0) pi = i;
  const DecBwdProblem& P = bt.p[pi];

  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int g = lane >> 4, c = lane & 15;
  u32x4* const Tw = w == 0 ? T0 : w == 1 ? T1 : w == 2 ? T2 : T3;
  const int M = bt.M, r = bt.r;
  const int N = P.N, K = P.K;                  // sizes fit 32 bits (N, K <= 2^21)
  const int nbr = K / 64;
  const int local = item - P.item0;
  const int cg = local / P.S, s = local - (local / P.S) * P.S;
  const int k0 = cg * kDwCols;
  const int nss = (N + kDwSS - 1) / kDwSS;
  const int ss0 = s * P.sps;
  const int nit = (ss0 + P.sps < nss ? ss0 + P.sps : nss) - ss0;

  // this lane's block; past K (a ragged last column group) its codes, scale
  // code and A values read as zero
  const int kb = cg * 4 + g;
  const bool kvalid = kQuad || kb < nbr;

  // the A rows of the LoRA term over the item's columns: thread t moves
  // chunks t and t + 256 of the 16 x 32 chunks of rank tile jt (row ci / 32,
  // logical chunk ci % 32); for one rank tile they are loaded now, during the
  // main loop's first loads, and used after it
  const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(NTU > 0 ? P.A : P.dy), 0, sgpr(NTU > 0 ? r * K * 2 : 0), kDbBufWord3);
  auto load_a = [&](int jt, int hh) {
    const int ci = 256 * hh + t, j = 16 * jt + (ci >> 5), kk = k0 + 8 * (ci & 31);
    const uint32_t ao = (j < r && kk < K) ? static_cast<uint32_t>((j * K + kk) * 2) : 0x80000000u;
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ars, ao, 0, 0));
  };
  u32x4 apre[2];
  if constexpr (NTU == 1) {
    apre[0] = load_a(0, 0);
    apre[1] = load_a(0, 1);
  }

  // ---- staging of dY (waves 0, 1) and of the B rows (waves 2, 3; r == 16) ----
  // Instruction h of wave w fills slots 256 (w % 2) + 64 h + lane. dY: slot =
  // row m * 32 + physical chunk, holding logical chunk phys ^ m of row m. B:
  // the super-step's 256 rows x 32 bytes are contiguous in memory and in LDS.
  // The super-step's first row sits in the descriptor's base; rows past M
  // (dY) or N (B) read as zero, and dY values past N are masked where used.
  uint32_t doff[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int slot = 256 * (w & 1) + 64 * h + lane;
    const int m = slot >> 5, phys = slot & 31;
    doff[h] = w < 2 ? static_cast<uint32_t>(m * N * 2 + (phys ^ m) * 16) : static_cast<uint32_t>(slot * 16);
  }
  auto dma_stage = [&](int ss, u32x4* ys, u32x4* bs) {
    const int n0 = ss * kDwSS;
    if (w < 2) {
      const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(P.dy + n0), 0, sgpr(M * N * 2 - n0 * 2), kDbBufWord3);
#pragma unroll
      for (int h = 0; h < 4; ++h)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(yr, (lds_void*)(ys + 256 * w + 64 * h), 16, doff[h], 0, 0, 0);
    } else if constexpr (kSB) {
      const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(P.B + static_cast<int64_t>(n0) * 16), 0, sgpr((N - n0) * 32), kDbBufWord3);
#pragma unroll
      for (int h = 0; h < 4; ++h)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(br, (lds_void*)(bs + 256 * (w - 2) + 64 * h), 16, doff[h], 0, 0,
                                                 0);
    }
  };
  const int ndma = (w < 2 || kSB) ? 4 : 0;     // wave-uniform

  // ---- this wave's operands of one super-step, loaded one ahead ----
  struct Codes {
    u32x4 cw[4][2];                            // chunk ch: block kb of row 64w + 16ch + c
    uint32_t q[kQuad ? 1 : 4];                 // ragged K: scale code byte and step per chunk
    float d[kQuad ? 1 : 4];
    u32x2 bu[4];                               // rank <= 16, r != 16: B[row][4g .. 4g + 3] per chunk
  };
  constexpr bool kPreB = !kSB && NTU == 1;
  const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(NTU > 0 ? P.B : P.dy), 0, sgpr(NTU > 0 ? N * r * 2 : 0), kDbBufWord3);
  const int64_t ngroups = (static_cast<int64_t>(N) * nbr + 255) >> 8;
  // B[n][16 jt + 4g .. + 3] (zero past N or r)
  auto load_b = [&](int n, int jt) {
    const int j = 16 * jt + 4 * g;
    const uint32_t bo = static_cast<uint32_t>((n * r + j) * 2);
    if ((r & 3) == 0)
      return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(brs, j < r ? bo : 0x80000000u, 0, 0));
    uint32_t h[4];                             // rows of B not 8-byte aligned: one rank at a time
#pragma unroll
    for (int e = 0; e < 4; ++e)
      h[e] = __builtin_amdgcn_raw_buffer_load_b16(brs, j + e < r ? bo + 2 * e : 0x80000000u, 0, 0);
    return u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
  };
  auto load_codes = [&](int ss, Codes& C) {
    const int nw0 = ss * kDwSS + 64 * w;       // the wave's first row
    const int rows = N - nw0 < 0 ? 0 : (N - nw0 < 64 ? N - nw0 : 64);
    const int nb = rows > 0 ? nw0 : 0;
    const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(P.packed + static_cast<int64_t>(nb) * (K / 2)), 0, sgpr(rows * (K / 2)), kDbBufWord3);
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      const uint32_t co = kvalid ? static_cast<uint32_t>((16 * ch + c) * (K / 2) + kb * 32) : 0x80000000u;
      C.cw[ch][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(crs, co, 0, 0));
      C.cw[ch][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(crs, co + 16, 0, 0));
    }
    if constexpr (!kQuad) {
      const int64_t sb = static_cast<int64_t>(nb) * nbr;
      const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<int8_t*>(P.qscale + sb), 0, sgpr(rows * nbr), kDbBufWord3);
      const int64_t g0 = sb >> 8;
      const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(P.step + g0), 0, sgpr(static_cast<int>((ngroups - g0) * 4)), kDbBufWord3);
#pragma unroll
      for (int ch = 0; ch < 4; ++ch) {
        const int bl = (16 * ch + c) * nbr + kb;
        C.q[ch] = __builtin_amdgcn_raw_buffer_load_b8(qrs, kvalid ? static_cast<uint32_t>(bl) : 0x80000000u, 0, 0);
        C.d[ch] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                srs, static_cast<uint32_t>((((sb & 255) + bl) >> 8) * 4), 0, 0));
      }
    }
    if constexpr (kPreB) {
#pragma unroll
      for (int ch = 0; ch < 4; ++ch) C.bu[ch] = load_b(nw0 + 16 * ch + c, 0);
    }
  };
  // the loads one load_codes issues with r % 4 == 0 (wave-uniform)
  constexpr int kCodeOps = 8 + (kQuad ? 0 : 8) + (kPreB ? 4 : 0);

  f32x4 acc[16], uacc[kU];
#pragma unroll
  for (int ct = 0; ct < 16; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int jt = 0; jt < kU; ++jt) uacc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // lane (g, c) reads rows 4g + c/4 of the tile, columns 16 ct + 4 (c % 4) ..
  // + 3, and receives column 16 ct + c of rows 4g .. 4g + 3
  const int rrow = 4 * g + (c >> 2);
  auto tr_off = [&](int ct) { return dw_slot(rrow, 2 * ct + ((c & 3) >> 1)) * 8 + 4 * (c & 1); };

  Codes c0, c1;
  if constexpr (kQuad) {
    // thread t loads the scale dword and step of row t of every super-step
    uint32_t qv[kDwMaxSps];
    float dv[kDwMaxSps];
#pragma unroll
    for (int u = 0; u < kDwMaxSps; ++u) {
      const int n = (ss0 + u) * kDwSS + t;
      const bool in = u < nit && n < N;
      const int64_t bl = static_cast<int64_t>(in ? n : 0) * nbr + 4 * cg;
      qv[u] = in ? *reinterpret_cast<const uint32_t*>(P.qscale + bl) : 0u;
      dv[u] = in ? P.step[bl >> 8] : 0.0f;
    }
    __builtin_amdgcn_sched_barrier(0);
    if (nit > 0) {                                 // the first super-step goes out behind them
      load_codes(ss0, c0);
      dma_stage(ss0, Y0, BS0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kDwMaxSps; ++u) {
      lq[u * kDwSS + t] = qv[u];
      ld[u * kDwSS + t] = dv[u];
    }
    sync();
  } else if (nit > 0) {
    load_codes(ss0, c0);
    dma_stage(ss0, Y0, BS0);
  }

  // iteration i: (1) every wave is past its reads of the staging buffers about
  // to be refilled (barrier); (2) request the next super-step; (3) wait until
  // this wave's staging loads of the current one have landed, then for all
  // waves' (barrier); (4) decode and multiply its four chunks. The waits are
  // explicit: the compiler does not track LDS written by direct loads.
  auto iter = [&](auto pre, int i, const Codes& cur, Codes& nxt, const u32x4* ys, const u32x4* bs, u32x4* ys_n,
                  u32x4* bs_n) {
    constexpr bool kPre = decltype(pre)::value;
    sync();
    if constexpr (kPre) {
      load_codes(ss0 + i + 1, nxt);
      dma_stage(ss0 + i + 1, ys_n, bs_n);
      __builtin_amdgcn_sched_barrier(0);
      // outstanding, oldest first: [codes i, stage i] [codes i+1, stage i+1]
      if (!kPreB || (r & 3) == 0) {
        if (ndma) wait_vm<kCodeOps + 4>();
        else wait_vm<kCodeOps>();
      } else {
        wait_vm<0>();
      }
    } else {
      wait_vm<0>();
    }
    sync();
    const int nrow0 = (ss0 + i) * kDwSS + 64 * w;     // the wave's first row of this super-step
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      float sc;
      if constexpr (kQuad) {
        const int ir = i * kDwSS + 64 * w + 16 * ch + c;
        sc = block_scale(static_cast<int8_t>(lq[ir] >> (8 * g)), ld[ir]);
      } else {
        sc = block_scale(static_cast<int8_t>(cur.q[ch]), cur.d[ch]);
      }
      const MagTable tb = make_table(cb, sc);
      const uint32_t pw[8] = {cur.cw[ch][0].x, cur.cw[ch][0].y, cur.cw[ch][0].z, cur.cw[ch][0].w,
                              cur.cw[ch][1].x, cur.cw[ch][1].y, cur.cw[ch][1].z, cur.cw[ch][1].w};
#pragma unroll
      for (int j = 0; j < 8; ++j) Tw[dw_slot(c, 8 * g + j)] = decode8_perm(pw[j], tb);
      // dY[c][rows 16ch + 4g .. + 3 of the wave's 64] (zero past N)
      const int nl = 64 * w + 16 * ch + 4 * g;
      const u32x2 yv = reinterpret_cast<const u32x2*>(ys)[dw_yslot(c, nl >> 3) * 2 + ((nl >> 2) & 1)];
      const s16x4 a = __builtin_bit_cast(s16x4, nrow0 + 16 * ch + 4 * g < N ? yv : u32x2{0u, 0u});
#pragma unroll
      for (int ct = 0; ct < 16; ++ct) acc[ct] = mfma16k16(a, ds_read_tr(Tw, tr_off(ct)), acc[ct]);
      if constexpr (kSB) {
        // staged B rows: row 64w + 16ch + rrow of the super-step, ranks
        // 4 (c % 4) .. + 3
        uacc[0] = mfma16k16(a, ds_read_tr(bs, (64 * w + 16 * ch + rrow) * 16 + 4 * (c & 3)), uacc[0]);
      } else if constexpr (NTU > 0) {
        // ranks beyond 16 are loaded here, for the chunk at hand
        u32x2* const U = UB[w];
#pragma unroll
        for (int jt = 0; jt < NTU; ++jt)
          U[jt * 64 + c * 4 + g] = kPreB ? cur.bu[ch] : load_b(nrow0 + 16 * ch + c, jt);
#pragma unroll
        for (int jt = 0; jt < NTU; ++jt)
          uacc[jt] = mfma16k16(
              a, ds_read_tr(reinterpret_cast<const u32x4*>(U), jt * 256 + rrow * 16 + 4 * (c & 3)), uacc[jt]);
      }
      // keep the next chunk's decode behind this chunk's multiplies (hoisting
      // it would hold its 64 decoded values in registers meanwhile)
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  using Pre = std::integral_constant<bool, true>;
  using NoPre = std::integral_constant<bool, false>;
  int i = 0;
  for (; i + 2 < nit; i += 2) {
    iter(Pre{}, i, c0, c1, Y0, BS0, Y1, BS1);
    iter(Pre{}, i + 1, c1, c0, Y1, BS1, Y0, BS0);
  }
  if (i + 1 < nit) {
    iter(Pre{}, i, c0, c1, Y0, BS0, Y1, BS1);
    iter(NoPre{}, i + 1, c1, c0, Y1, BS1, Y0, BS0);
  } else if (i < nit) {
    iter(NoPre{}, i, c0, c1, Y0, BS0, Y1, BS1);
  }

  // ---- the four waves' parts, summed in wave order ----
  __syncthreads();
  if constexpr (NTU > 0) {
    // u_s: lane (g, c) of rank tile jt holds u[4 g + v][16 jt + c]
#pragma unroll
    for (int jt = 0; jt < NTU; ++jt) Tw[jt * 64 + lane] = __builtin_bit_cast(u32x4, uacc[jt]);
    __syncthreads();
    if (w == 0) {
#pragma unroll
      for (int jt = 0; jt < NTU; ++jt) {
        const int idx = jt * 64 + lane;
        f32x4 u = __builtin_bit_cast(f32x4, T0[idx]);
        u += __builtin_bit_cast(f32x4, T1[idx]);
        u += __builtin_bit_cast(f32x4, T2[idx]);
        u += __builtin_bit_cast(f32x4, T3[idx]);
#pragma unroll
        for (int v = 0; v < 4; ++v) Ush[(4 * g + v) * (16 * kU) + 16 * jt + c] = u[v];
      }
    }
    __syncthreads();
  }
  // accumulators: round h moves tiles 8h .. 8h + 7 through the four tiles'
  // memory; wave w keeps the sums of tiles 8h + 2w and 8h + 2w + 1
  f32x4 fin[4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int e = 0; e < 8; ++e) Tw[e * 64 + lane] = __builtin_bit_cast(u32x4, acc[8 * h + e]);
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int idx = (2 * w + e) * 64 + lane;
      f32x4 v = __builtin_bit_cast(f32x4, T0[idx]);
      v += __builtin_bit_cast(f32x4, T1[idx]);
      v += __builtin_bit_cast(f32x4, T2[idx]);
      v += __builtin_bit_cast(f32x4, T3[idx]);
      fin[2 * h + e] = v;
    }
    __syncthreads();
  }
  // fin[f] is tile ct_of(f) = 8 (f / 2) + 2 w + (f % 2)
  auto ct_of = [&](int f) { return 8 * (f >> 1) + 2 * w + (f & 1); };

  if constexpr (NTU > 0) {
#pragma unroll
    for (int jt = 0; jt < NTU; ++jt) {
      // (alpha/r) u_s as hi + lo bf16: the A operand, lane (g, c) holding
      // ranks 16 jt + 4g .. + 3 of row m = c
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = bt.scale * Ush[c * (16 * kU) + 16 * jt + 4 * g + e];
      const uint32_t h0 = pack_bf16x2(v[0], v[1]), h1 = pack_bf16x2(v[2], v[3]);
      const uint32_t l0 = pack_bf16x2(v[0] - bf16_lo(h0), v[1] - bf16_hi(h0));
      const uint32_t l1 = pack_bf16x2(v[2] - bf16_lo(h1), v[3] - bf16_hi(h1));
      // A rows 16 jt .. 16 jt + 15 over the item's columns, in the tile's
      // column order, staged in T0
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int ci = 256 * hh + t;
        T0[dw_slot(ci >> 5, ci & 31)] = perm8(NTU == 1 ? apre[hh] : load_a(jt, hh));
      }
      __syncthreads();
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const s16x4 b = ds_read_tr(T0, tr_off(ct_of(f)));
        fin[f] = mfma16k16(__builtin_bit_cast(s16x4, u32x2{h0, h1}), b, fin[f]);
        fin[f] = mfma16k16(__builtin_bit_cast(s16x4, u32x2{l0, l1}), b, fin[f]);
      }
      __syncthreads();
    }
  }

  // lane (g, c) of tile ct holds dX[4 g + v][k0 + db_col(16 ct + c)]
  if (P.S == 1) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int k = k0 + db_col(16 * ct_of(f) + c);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 4 * g + v;
        if (m < M && k < K) P.dx[static_cast<int64_t>(m) * K + k] = bf16_bits(fin[f][v]);
      }
    }
    return;
  }
  // split rows: partial sums [256 positions][Mp] of this split, then the last
  // split of the column group to arrive adds all of them in split order
  // (device-scope coherent stores and loads, the arrival counter as in the
  // decode-shaped forward)
  const int Mp = (M + 3) & ~3;
  float* const part_cg = bt.part + (P.part0 + static_cast<int64_t>(cg) * P.S) * (kDwCols * Mp);
  const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
      part_cg, 0, sgpr(P.S * kDwCols * Mp * 4), kDbBufWord3);
  if (4 * g < M) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const uint32_t off = static_cast<uint32_t>(((s * kDwCols + 16 * ct_of(f) + c) * Mp + 4 * g) * 4);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, fin[f]), prs, off, 0, 16);
    }
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);                  // this wave's stores have completed
  __syncthreads();
  if (t == 0) {
    const unsigned old = __hip_atomic_fetch_add(bt.cnt + P.cnt0 + cg, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    last_flag = old == static_cast<unsigned>(P.S - 1);
  }
  __syncthreads();
  if (!last_flag) return;
  // thread t adds the four-value groups t, t + 256, t + 512, t + 768 (position
  // p, rows m0 .. m0 + 3) over the splits, four splits' loads of all its
  // groups in flight at a time
  const int ngr = kDwCols * Mp / 4;               // 256 .. 1024 groups
  f32x4 sum[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) sum[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int sp0 = 0; sp0 < P.S; sp0 += 4) {
    f32x4 v[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i4 = t + 256 * e;
        const uint32_t off = static_cast<uint32_t>(((sp0 + u) * kDwCols * Mp + 4 * i4) * 4);
        v[u][e] = (sp0 + u < P.S && i4 < ngr)
                      ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(prs, off, 0, 16))
                      : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) sum[e] += v[u][e];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i4 = t + 256 * e;
    if (i4 < ngr) {
      const int p = 4 * i4 / Mp, m0 = 4 * i4 - p * Mp;
      const int k = k0 + db_col(p);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (m0 + q < M && k < K) P.dx[static_cast<int64_t>(m0 + q) * K + k] = bf16_bits(sum[e][q]);
    }
  }
  if (t == 0) __hip_atomic_store(bt.cnt + P.cnt0 + cg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
namespace {

// narrow items: about kDbTargetItems per launch, at least kDbMinSps sub-tiles
// of 64 rows per split
DecChunkPlan plan_narrow(int cn, const int64_t* N, const int64_t* K) {
  DecChunkPlan pl;
  int64_t cols = 0;
  for (int i = 0; i < cn; ++i) cols += K[i] / kDnCols;
  const int64_t s_all = cols >= kDbTargetItems / 2 ? 1 : cdiv(kDbTargetItems, cols);
  for (int i = 0; i < cn; ++i) {
    const int64_t nst = cdiv(N[i], kDnSub);
    int64_t S = cdiv(nst, kDbMinSps);
    if (S > s_all) S = s_all;
    if (S < 1) S = 1;
    const int64_t sps = cdiv(nst, S);
    S = cdiv(nst, sps);
    const int64_t kbs = K[i] / kDnCols;
    pl.S[i] = static_cast<int>(S);
    pl.sps[i] = static_cast<int>(sps);
    pl.items += kbs * S;
    if (S > 1) {
      pl.slots += kbs * S;
      pl.counters += kbs;
    }
  }
  return pl;
}

// wide items: about kDbWideTarget per launch, at most kDwMaxSps super-steps
// each; with more split column ranges than the workspace has arrival counters
// for, every weight runs unsplit (the launch then has items enough)
DecChunkPlan plan_wide(int cn, const int64_t* N, const int64_t* K) {
  int64_t cgs_all = 0;
  for (int i = 0; i < cn; ++i) cgs_all += cdiv(K[i], kDwCols);
  const int64_t s_all = cgs_all >= kDbWideTarget / 2 ? 1 : cdiv(kDbWideTarget, cgs_all);
  for (int bounded = 1; bounded >= 0; --bounded) {
    DecChunkPlan pl;
    pl.wide = true;
    for (int i = 0; i < cn; ++i) {
      const int64_t nss = cdiv(N[i], kDwSS);
      int64_t S = 1, sps = nss;
      if (bounded) {
        S = s_all < nss ? s_all : nss;
        sps = cdiv(nss, S);
        if (sps > kDwMaxSps) sps = kDwMaxSps;
        S = cdiv(nss, sps);
      }
      const int64_t cgs = cdiv(K[i], kDwCols);
      pl.S[i] = static_cast<int>(S);
      pl.sps[i] = static_cast<int>(sps);
      pl.items += cgs * S;
      if (S > 1) {
        pl.slots += cgs * S;
        pl.counters += cgs;
      }
    }
    if (!bounded || pl.counters * 4 <= static_cast<int64_t>(kWsCounterBytes)) return pl;
  }
  return DecChunkPlan{};
}

}  // namespace

DecChunkPlan dec_bwd_plan_chunk(int64_t M, int cn, const int64_t* N, const int64_t* K) {
  (void)M;
  int64_t cgs_all = 0;
  for (int i = 0; i < cn; ++i) cgs_all += cdiv(K[i], kDwCols);
  return cgs_all >= kDbWideMin ? plan_wide(cn, N, K) : plan_narrow(cn, N, K);
}

size_t dec_bwd_workspace_bytes(int64_t M, int G, const int64_t* N, const int64_t* K) {
  size_t most = 0;
  const int64_t Mp = round_up(M, 4);
  for (int c0 = 0; c0 < G; c0 += kDecMaxProblems) {
    const int cn = G - c0 < kDecMaxProblems ? G - c0 : kDecMaxProblems;
    const DecChunkPlan pl = dec_bwd_plan_chunk(M, cn, N + c0, K + c0);
    const size_t b = static_cast<size_t>(pl.slots * (pl.wide ? kDwCols : kDnCols) * Mp * 4);
    if (b > most) most = b;
  }
  return most ? kWsCounterBytes + align256(most) : 0;
}

hipError_t launch_dec_bwd(int64_t M, int G, const uint16_t* const* dy, const int64_t* N, const int64_t* K,
                          const uint8_t* const* packed, const int8_t* const* qscale, const float* const* step,
                          const uint16_t* const* A, const uint16_t* const* B, int r, float alpha,
                          uint16_t* const* dx, void* ws, const Codebook& cb, hipStream_t stream) {
  char* wsb = static_cast<char*>(ws);
  const int NT = r <= 0 ? 0 : r <= 16 ? 1 : r <= 32 ? 2 : r <= 64 ? 4 : 8;
  mark_kernel(0, stream);
  for (int c0 = 0; c0 < G; c0 += kDecMaxProblems) {
    const int cn = G - c0 < kDecMaxProblems ? G - c0 : kDecMaxProblems;
    const DecChunkPlan pl = dec_bwd_plan_chunk(M, cn, N + c0, K + c0);
    const int cols = pl.wide ? kDwCols : kDnCols;
    DecBwdBatch bt{};
    bt.count = cn;
    bt.M = static_cast<int>(M);
    bt.r = r;
    bt.scale = r > 0 ? alpha / static_cast<float>(r) : 0.0f;
    bt.cnt = pl.slots ? reinterpret_cast<unsigned*>(wsb) : nullptr;
    bt.part = pl.slots ? reinterpret_cast<float*>(wsb + kWsCounterBytes) : nullptr;
    int items = 0, slot = 0, cnt = 0;
    bool quad = true;
    for (int i = 0; i < cn; ++i) {
      const int q = c0 + i;
      DecBwdProblem& P = bt.p[i];
      P.dy = dy[q];
      P.packed = packed[q];
      P.qscale = qscale[q];
      P.step = step[q];
      P.A = r > 0 ? A[q] : nullptr;
      P.B = r > 0 ? B[q] : nullptr;
      P.dx = dx[q];
      P.N = static_cast<int>(N[q]);
      P.K = static_cast<int>(K[q]);
      P.S = pl.S[i];
      P.sps = pl.sps[i];
      P.item0 = items;
      const int cgs = static_cast<int>(cdiv(K[q], cols));
      items += cgs * P.S;
      P.part0 = slot;
      P.cnt0 = cnt;
      if (P.S > 1) {
        slot += cgs * P.S;
        cnt += cgs;
      }
      quad = quad && K[q] % 256 == 0;
    }
    bt.items = items;
    const dim3 grid(static_cast<unsigned>(round_up(items, 8))), block(64 * kDbWaves);
    if (!pl.wide) {
#define QNF4_DN(NTV) hipLaunchKernelGGL(HIP_KERNEL_NAME(k_dec_bwd_narrow<NTV>), grid, block, 0, stream, bt, cb)
      switch (NT) {
        case 0: QNF4_DN(0); break;
        case 1: QNF4_DN(1); break;
        case 2: QNF4_DN(2); break;
        case 4: QNF4_DN(4); break;
        default: QNF4_DN(8); break;
      }
#undef QNF4_DN
    } else {
#define QNF4_DW(NTV, SBV)                                                                                  \
  if (quad)                                                                                                \
    hipLaunchKernelGGL(HIP_KERNEL_NAME(k_dec_bwd_wide<NTV, SBV, true>), grid, block, 0, stream, bt, cb); \
  else                                                                                                     \
    hipLaunchKernelGGL(HIP_KERNEL_NAME(k_dec_bwd_wide<NTV, SBV, false>), grid, block, 0, stream, bt, cb)
      switch (NT) {
        case 0: QNF4_DW(0, false); break;
        case 1:
          if (r == 16) {
            QNF4_DW(1, true);
          } else {
            QNF4_DW(1, false);
          }
          break;
        case 2: QNF4_DW(2, false); break;
        case 4: QNF4_DW(4, false); break;
        default: QNF4_DW(8, false); break;
      }
#undef QNF4_DW
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  mark_kernel(1, stream);
  return hipSuccess;
}

}  // namespace qnf4
