// Decode-shaped (M <= 16) fused NF4-dequant backward for gfx950, over a table
// of weights in one launch.
//
//   dX_p = bf16( dY_p . W_p' + (alpha/r) . u_p . A_p ),  u_p = dY_p . B_p
//
// for every weight p of the table ("A 65B fine-tune on the GPU you already
// have", figure 2: the gradient flows through the frozen weights, which become
// bf16 block by block right before the multiply; "QLoRA" (techbytebybyte),
// "Follow one QLoRA training step"). At these shapes each weight is used by at
// most 16 rows, so the kernel streams the 0.516 bytes/param stored weight once
// and is bound by that stream and by the VALU work of decoding it.
//
// Work items. An item is one 64-column block column of dX x a range of W's
// rows, run by one workgroup of four waves that take the item's 64-row
// sub-tiles in turn. N is split into S row ranges when the launch has too few
// block columns to fill the chip; every split writes fp32 partial sums and the
// last split of a block column to arrive (an arrival counter in the workspace)
// adds them in split order, so results do not depend on scheduling. Items of
// one block column run on one XCD (consecutive workgroup ids go round robin
// over the 8 XCDs), so their partials stay in that XCD's L2, and the four
// block columns that share the 128-byte lines of a weight row run side by side
// there.
//
// Sub-tile (64 rows x 64 columns). Lane (g, c) of a wave loads the 32 code
// bytes of row 16g + c, decodes them with the block's table into 64 bf16 and
// writes them to the wave's own LDS tile. The contraction runs over W's rows,
// so the B operands of the 16x16x32 MFMAs (8 rows of one column) are read back
// transposed (ds_read_b64_tr_b16), against dY[c][8 rows]. The tile is private
// to the wave and a wave's LDS operations complete in order, so the main loop
// has no workgroup barrier. The operands of the next sub-tile are loaded while
// the current one is decoded and multiplied.
//
// LoRA. The B rows of each sub-tile go through the same transposed path, so
// the item also accumulates u_s = dY . B over its own rows. After the main
// loop the four waves' parts of the partial sums and of u_s are added through
// LDS (fixed order), and (alpha/r) . u_s . A over the item's columns is added
// with (alpha/r) . u_s carried as the sum of two bf16 values (hi + lo, about 16
// significant bits), so splitting N leaves the LoRA term exact to fp32-level
// rounding instead of requiring the full u before any output.
//
// Decode order. decode8_perm yields the 8 weights of a code dword in the order
// 0 2 4 6 1 3 5 7; the tile's columns keep that order (the A rows of the LoRA
// term are permuted the same way), and the outputs go to their true columns.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mm_common.hpp"

namespace qnf4 {

constexpr int kDbWaves = 4;
constexpr int kDbCols = 64;                    // dX columns per item (one block column)
constexpr int kDbSub = 64;                     // weight rows per sub-tile
constexpr int kDbUChunks = 192;                // 16-byte chunks of one rank tile's B rows (padded)
constexpr int kDbBufWord3 = 0x00020000;        // raw buffer descriptor word 3 on gfx9-family parts

// 16-byte chunk ch (0..7) of row `row` (0..63) of the 64 x 64 bf16 tile. The
// writes (16 lanes: 16 consecutive rows, one chunk) and the transposed reads
// (32 lanes: 8 rows, two adjacent chunks) each touch all 64 banks once.
__device__ __forceinline__ int db_slot(int row, int ch) {
  const int i = (row >> 1) & 7;
  return row * 8 + (ch ^ (((i & 1) << 1) | ((i >> 1) & 1) | (i & 4)));
}
// chunk ch (0, 1) of row `row` of the B rows of one rank tile (16 ranks); a
// chunk of padding after every 8 rows keeps the transposed reads conflict-free
__device__ __forceinline__ int db_uslot(int row, int ch) { return row * 2 + ch + 8 * (row >> 3); }

// position p of a decoded 8-group holds element pi(p) (order 0 2 4 6 1 3 5 7)
__device__ __forceinline__ int db_col(int p) { return (p & ~7) | ((p & 3) << 1) | ((p >> 2) & 1); }

__device__ __forceinline__ f32x4 mfma16k16(const s16x4& a, const s16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int db_item_of(int wg, int grid) {
  // grid is a multiple of 8: XCD (wg % 8) gets items [xcd * grid/8, ...)
  return (wg & 7) * (grid >> 3) + (wg >> 3);
}

// B operand of a 16x16x32 MFMA (rows row0 .. row0 + 7 of a tile, column
// col0 + c) from the decoded tile (kU = false) or the B rows of a rank tile
// (kU = true): two transposed 8-byte reads, rows row0 + 4q + c/4, columns
// col0 + 4 (c % 4) .. + 3
template <bool kU>
__device__ __forceinline__ bf16x8 tr_operand(const u32x4* base, int row0, int col0, int c) {
  s16x4 v[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int row = row0 + 4 * q + (c >> 2), col = col0 + 4 * (c & 3);
    const int sl = kU ? db_uslot(row, col >> 3) : db_slot(row, col >> 3);
    v[q] = ds_read_tr(base, sl * 8 + (col & 4));
  }
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// NTU: rank tiles of 16 (0: no adapter; else a power of two with 16 NTU >= r).
template <int NTU>
__global__ __launch_bounds__(64 * kDbWaves, 3) void k_dec_bwd(DecBwdBatch bt, Codebook cb) {
  constexpr int kU = NTU > 0 ? NTU : 1;
  // per wave: the decoded sub-tile (8 KB; then its accumulators for the
  // cross-wave sums, then the A rows of its LoRA term) and the B rows of a
  // sub-tile (then its part of u_s, then u_s)
  __shared__ u32x4 T0[512], T1[512], T2[512], T3[512];
  __shared__ u32x4 U0[kDbUChunks * kU], U1[kDbUChunks * kU], U2[kDbUChunks * kU], U3[kDbUChunks * kU];
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
  const int nst = (N + kDbSub - 1) / kDbSub;
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
    const int n0 = st * kDbSub;
    const int rows = N - n0 < kDbSub ? N - n0 : kDbSub;
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
    for (int j = 0; j < 8; ++j) Tw[db_slot(row, j)] = decode8_perm(pw[j], tb);
    if constexpr (NTU > 0) {
#pragma unroll
      for (int jt = 0; jt < NTU; ++jt)
#pragma unroll
        for (int h = 0; h < 2; ++h) Uw[kDbUChunks * jt + db_uslot(row, h)] = S.bu[jt][h];
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 a = as_bf16x8(S.dyf[ks]);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, tr_operand<false>(Tw, 32 * ks + 8 * g, 16 * ct, c),
                                                          acc[ct], 0, 0, 0);
      if constexpr (NTU > 0) {
#pragma unroll
        for (int jt = 0; jt < NTU; ++jt)
          uacc[jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              a, tr_operand<true>(Uw + kDbUChunks * jt, 32 * ks + 8 * g, 0, c), uacc[jt], 0, 0, 0);
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
      if (lane < 32) Tw[db_slot(lane >> 1, 2 * w + (lane & 1))] = perm8(apre[jt]);
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = bt.scale * ush[c * (16 * kU) + 16 * jt + 4 * g + e];
      const uint32_t h0 = pack_bf16x2(v[0], v[1]), h1 = pack_bf16x2(v[2], v[3]);
      const uint32_t l0 = pack_bf16x2(v[0] - bf16_lo(h0), v[1] - bf16_hi(h0));
      const uint32_t l1 = pack_bf16x2(v[2] - bf16_lo(h1), v[3] - bf16_hi(h1));
      // B operand: ranks 4g .. 4g + 3 (rows of the staged A) of column 16 w + c
      const int rr = 4 * g + (c >> 2), col = 16 * w + 4 * (c & 3);
      const s16x4 b = ds_read_tr(Tw, db_slot(rr, col >> 3) * 8 + (col & 4));
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
  float* const part_kb = bt.part + (P.part0 + static_cast<int64_t>(kb) * P.S) * (kDbCols * Mp);
  const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
      part_kb, 0, P.S * kDbCols * Mp * 4, kDbBufWord3);
  if (4 * g < M) {
    const uint32_t off = static_cast<uint32_t>(((s * kDbCols + 16 * w + c) * Mp + 4 * g) * 4);
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
  if (t < kDbCols * Mp / 4) {
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
    for (int sp0 = 0; sp0 < P.S; sp0 += 8) {
      f32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t off = static_cast<uint32_t>(((sp0 + u) * kDbCols * Mp + 4 * t) * 4);
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

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
DecChunkPlan dec_bwd_plan_chunk(int64_t M, int cn, const int64_t* N, const int64_t* K) {
  (void)M;
  DecChunkPlan pl;
  int64_t cols = 0;
  for (int i = 0; i < cn; ++i) cols += K[i] / kDbCols;
  // about kDbTargetItems items per launch; a split covers at least kDbMinSps
  // sub-tiles (each split costs a round of fp32 partials and a fix-up)
  const int64_t s_all = cols >= kDbTargetItems / 2 ? 1 : cdiv(kDbTargetItems, cols);
  for (int i = 0; i < cn; ++i) {
    const int64_t nst = cdiv(N[i], kDbSub);
    int64_t S = cdiv(nst, kDbMinSps);
    if (S > s_all) S = s_all;
    if (S < 1) S = 1;
    const int64_t sps = cdiv(nst, S);
    S = cdiv(nst, sps);
    const int64_t kbs = K[i] / kDbCols;
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

size_t dec_bwd_workspace_bytes(int64_t M, int G, const int64_t* N, const int64_t* K) {
  int64_t max_slots = 0;
  for (int c0 = 0; c0 < G; c0 += kDecMaxProblems) {
    const int cn = G - c0 < kDecMaxProblems ? G - c0 : kDecMaxProblems;
    const DecChunkPlan pl = dec_bwd_plan_chunk(M, cn, N + c0, K + c0);
    if (pl.slots > max_slots) max_slots = pl.slots;
  }
  if (max_slots == 0) return 0;
  const int64_t Mp = round_up(M, 4);
  return kWsCounterBytes + align256(static_cast<size_t>(max_slots * kDbCols * Mp * 4));
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
    DecBwdBatch bt{};
    bt.count = cn;
    bt.M = static_cast<int>(M);
    bt.r = r;
    bt.scale = r > 0 ? alpha / static_cast<float>(r) : 0.0f;
    bt.cnt = pl.slots ? reinterpret_cast<unsigned*>(wsb) : nullptr;
    bt.part = pl.slots ? reinterpret_cast<float*>(wsb + kWsCounterBytes) : nullptr;
    int items = 0, slot = 0, cnt = 0;
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
      const int kbs = static_cast<int>(K[q] / kDbCols);
      items += kbs * P.S;
      P.part0 = slot;
      P.cnt0 = cnt;
      if (P.S > 1) {
        slot += kbs * P.S;
        cnt += kbs;
      }
    }
    bt.items = items;
    const dim3 grid(static_cast<unsigned>(round_up(items, 8)));
#define QNF4_DB(NTV) hipLaunchKernelGGL(HIP_KERNEL_NAME(k_dec_bwd<NTV>), grid, dim3(64 * kDbWaves), 0, stream, bt, cb)
    switch (NT) {
      case 0: QNF4_DB(0); break;
      case 1: QNF4_DB(1); break;
      case 2: QNF4_DB(2); break;
      case 4: QNF4_DB(4); break;
      default: QNF4_DB(8); break;
    }
#undef QNF4_DB
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  mark_kernel(1, stream);
  return hipSuccess;
}

}  // namespace qnf4
