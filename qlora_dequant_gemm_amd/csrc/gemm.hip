// Fused NF4-dequant matmuls for gfx950 (MI355X).
//
// Forward  y  = bf16( x . W'^T + (alpha/r) . t . B^T ),  t = bf16(x . A^T)
// Backward dX = bf16( dY . W'  + (alpha/r) . u . A   ),  u = bf16(dY . B)
// with W' the bf16 dequantization of the NF4 weight, done block by block
// right before the multiply ("A 65B fine-tune on the GPU you already have",
// figure 2; "QLoRA Explained", "What is QLoRA?").
//
// Kernels (M > 16; the decode shapes have their own kernels)
//   k_gemm_fwd    M > 16: 256x256 output tile, 4 waves each owning 64 output
//                 columns; each lane dequantizes its MFMA B operands straight
//                 into registers, x goes through double-buffered LDS; 32x32x16
//                 bf16 MFMA with fp32 accumulation; LoRA as a rank-r MFMA in
//                 the epilogue. MFMA-bound.
//   k_gemm_bwd    M > 16: same tiling over dX [M, K]; the contraction runs over
//                 W's rows, so the dequantized tile is stored row-major and
//                 read transposed with ds_read_b64_tr_b16.
// The rank-r down projections t and u come from k_down_rows (lora.hip).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "mm_common.hpp"

namespace qnf4 {

// ---------------------------------------------------------------------------
// Tiled MFMA GEMMs (M > 16)
// ---------------------------------------------------------------------------
constexpr int kTile = 256;
constexpr int kChunks = 2048;                // 16-byte chunks in one 256x64 bf16 tile

// Workgroup id -> output tile. Consecutive ids land on different XCDs (round
// robin over 8), so each XCD is first given a contiguous range of the tile
// order; that order then sweeps groups of 4 tile-rows across all tile-columns
// so co-resident workgroups share operand tiles in their XCD's L2 (the 32
// workgroups an XCD runs at once cover 4 x 8 tiles: a quarter less L2 fill
// than 8 x 4, since an x tile row is four times the bytes of a code column).
__device__ __forceinline__ void tile_of(int pid, int ntm, int ntn, int& tm, int& tn) {
  const int total = ntm * ntn;
  int p = pid;
  if ((total & 7) == 0) p = (pid & 7) * (total >> 3) + (pid >> 3);
  const int G = 4;
  const int group = p / (G * ntn);
  const int first_m = group * G;
  const int gsz = (ntm - first_m) < G ? (ntm - first_m) : G;
  const int within = p - group * G * ntn;
  tm = first_m + within % gsz;
  tn = within / gsz;
}

// A tile (256 rows x 64 deep, bf16) in LDS: row-major, 8 chunks of 16 bytes
// per row. The LDS has 64 four-byte banks and serves a 16-byte-per-lane read
// 16 lanes at a time; a 128-byte row covers half the banks, so rows of one
// parity share a half. Logical chunk c of row r sits at physical chunk
// c ^ ((r >> 1) & 7): 16 consecutive rows reading the same logical chunk then
// land on 8 distinct chunks in each half, i.e. on all 64 banks once.
__device__ __forceinline__ int a_swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int a_slot(int row, int ch) { return row * 8 + (ch ^ a_swz(row)); }

// ---------------------------------------------------------------------------
// k_gemm_fwd: y [M, N] = x . W'^T (+ LoRA), M > 16.
//
// Workgroup tile 256 (M) x 256 (N), 4 waves; wave w owns output columns
// [64w, 64w + 64) for all 256 rows: 8 x 2 blocks of 32x32x16 bf16 MFMA with
// fp32 accumulators. In this NT layout one packed dword (8 codes of one
// weight row) is exactly one MFMA B operand, so each lane dequantizes its own
// B operands straight into registers and every weight is decoded once.
//
// Memory traffic is what limits this kernel, so every stream is moved in
// whole 128-byte lines:
//   x      global -> LDS by DMA (buffer_load ... lds), a ring of four 256x64
//          tiles; the tile of step k+3 is requested at the start of step k.
//   codes  each wave DMAs the codes of its own 64 weight rows for a super-step
//          of four K steps (64 rows x 128 bytes = 8 KB) into a private LDS
//          slab; lanes then read their 16-byte code words from LDS. The slab
//          of super-step S+1 is requested in step 4S+2, right after that
//          step has read the last codes of super-step S.
//   scales q and d of step k+2 are loaded at the start of step k.
// In step k the MFMAs of step k run while the codes of step k+1 are decoded.
// LDS: 4 x 32 KB of x + 4 x 8 KB of codes = 160 KB, one workgroup per CU.
//
// K permutation: within a step, lane half h holds k in [32h, 32h + 32) and
// MFMA sub-step s uses k = 32h + 8s + (0..7) on both operands (the sum over k
// is order-free), so a lane's codes for a step are one 16-byte word.
// ---------------------------------------------------------------------------
constexpr int kBufferDword3 = 0x00020000;    // raw buffer descriptor word 3 on gfx9-family parts

struct BScale {
  float d[2];      // second-level steps of this lane's weight rows (N-blocks j)
  int8_t q[2];     // block scale codes
  float live;      // 1 for a real K step, 0 for a step past the end
};
struct BScale4 {   // the same for the four steps of a super-step
  float d[2];
  uint32_t q[2];   // byte u = scale code of step 4S + u
};


// kQuad: K is a multiple of 256, so the four block-scale codes of a
// super-step are one aligned 4-byte word of qscale and share one second-level
// step (a 256-block group never splits 4-aligned blocks); scales are then
// loaded once per super-step. Otherwise they are loaded per step.
// RSN: chunks of 16 ranks in the LoRA epilogue (1 for r <= 16: t's padding
// columns 16 .. 31 are zero and skipped; else rank_pad(r) / 16), 0 for none.
template <bool kQuad, int RSN>
__global__ __launch_bounds__(256, 1) void k_gemm_fwd(FwdTable tab, int64_t M, int rp, int r, float scale,
                                                     Codebook cb) {
  // ring of four x tiles (32 KB each) and the per-wave code slabs (8 KB each),
  // distinct objects so that the compiler can tell a DMA into one from reads
  // of another
  __shared__ u32x4 As0[kChunks];
  __shared__ u32x4 As1[kChunks];
  __shared__ u32x4 As2[kChunks];
  __shared__ u32x4 As3[kChunks];
  __shared__ u32x4 Bs[4 * 512];
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);   // wave index, provably uniform (SGPR)
  const int h = lane >> 5, l32 = lane & 31;
  // The weights' tile columns are numbered one after another, so the tile
  // order sweeps groups of tile-rows across every weight of the table (x
  // rows shared by weights with the same input stay in L2 across them).
  const int ntm = static_cast<int>(cdiv(M, kTile));
  int tm, tnv;
  tile_of(blockIdx.x, ntm, tab.col0[tab.count], tm, tnv);
  tm = __builtin_amdgcn_readfirstlane(tm);     // uniform already; this keeps the
  tnv = __builtin_amdgcn_readfirstlane(tnv);   // buffer descriptors in SGPRs
  int g = 0;
#pragma unroll
  for (int i = 1; i < kFwdMaxWeights; ++i)
    if (i < tab.count && tnv >= tab.col0[i]) g = i;
  g = __builtin_amdgcn_readfirstlane(g);
  const int tn = tnv - tab.col0[g];
  const uint16_t* __restrict__ x = tab.x[g];
  const uint8_t* __restrict__ packed = tab.packed[g];
  const int8_t* __restrict__ qscale = tab.qscale[g];
  const float* __restrict__ step = tab.step[g];
  const uint16_t* __restrict__ tl = tab.tl[g];
  const uint16_t* __restrict__ Bl = tab.B[g];
  uint16_t* __restrict__ y = tab.y[g];
  const int64_t N = tab.N[g], K = tab.K[g];
  const int64_t m0 = static_cast<int64_t>(tm) * kTile, n0 = static_cast<int64_t>(tn) * kTile;
  const int64_t nk = K / 64;
  const int64_t nsup = (nk + 3) / 4;           // super-steps of four K steps

  // x tile DMA (rows past M read as zero through the descriptor's range
  // check). Instruction i of wave w fills LDS rows 64w + 8i + (lane >> 3),
  // physical chunk lane & 7, i.e. logical chunk (lane & 7) ^ a_swz(row); the
  // K step goes in soffset.
  const int64_t rows_valid = imin(static_cast<int64_t>(kTile), M - m0);
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x + m0 * K), 0, static_cast<int>(rows_valid * K * 2), kBufferDword3);
  uint32_t voff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 64 * w + 8 * i + (lane >> 3);
    voff[i] = static_cast<uint32_t>(row * K * 2 + 16 * ((lane & 7) ^ a_swz(row)));
  }
  auto dma_a = [&](int64_t kt, u32x4* Ab) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      lds_void* dst = (lds_void*)(&Ab[(64 * w + 8 * i) * 8]);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, dst, 16, voff[i], static_cast<uint32_t>(kt * 128), 0, 0);
    }
  };
  // code slab DMA: wave w's rows n0 + 64w + r, r = 8i + (lane >> 3), bytes
  // [128 S, 128 S + 128) of each packed row, same chunk swizzle as x. A
  // super-step past the end re-reads the last one (its steps are dead).
  const int64_t nrows_valid = imin(static_cast<int64_t>(kTile), N - n0);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(packed + n0 * (K / 2)), 0, static_cast<int>(nrows_valid * (K / 2)), kBufferDword3);
  uint32_t boff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r8 = 8 * i + (lane >> 3);
    boff[i] = static_cast<uint32_t>((64 * w + r8) * (K / 2) + 16 * ((lane & 7) ^ a_swz(r8)));
  }
  u32x4* const Bw = Bs + 512 * w;              // this wave's slab: 64 rows x 8 chunks
  auto dma_b = [&](int64_t S) {
    const uint32_t so = static_cast<uint32_t>(imin(S, nsup - 1) * 128);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      lds_void* dst = (lds_void*)(&Bw[64 * i]);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, dst, 16, boff[i], so, 0, 0);
    }
  };
  // the 16-byte code words of K step kt for this lane (N-blocks j = 0, 1)
  auto read_codes = [&](int64_t kt, u32x4 (&c)[2]) {
    const int ch = (2 * static_cast<int>(kt & 3) + h) ^ a_swz(l32);   // a_swz(32 j + l32) == a_swz(l32)
#pragma unroll
    for (int j = 0; j < 2; ++j) c[j] = Bw[(32 * j + l32) * 8 + ch];
  };
  int64_t bblk[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) bblk[j] = imin(n0 + 64 * w + 32 * j + l32, N - 1) * nk;
  // block scales of K step kt; a step past the end (the loop runs whole
  // super-steps) re-reads the last one and is marked dead, which makes its
  // block scale, and so every decoded weight, zero
  auto load_s = [&](int64_t kt, BScale& P) {
    const int64_t kc = imin(kt, nk - 1);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      P.q[j] = qscale[bblk[j] + kc];
      P.d[j] = step[(bblk[j] + kc) >> 8];
    }
    P.live = kt < nk ? 1.0f : 0.0f;
  };
  auto load_s4 = [&](int64_t S, BScale4& P) {
    const int64_t kc = 4 * imin(S, nsup - 1);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      P.q[j] = *reinterpret_cast<const uint32_t*>(qscale + bblk[j] + kc);
      P.d[j] = step[(bblk[j] + kc) >> 8];
    }
  };
  // scales of step kt (position u in its super-step) from a quad
  auto scale_of = [&](const BScale4& P, int u, int64_t kt, int j) {
    const int8_t q = static_cast<int8_t>((P.q[j] >> (8 * u)) & 0xFFu);
    return block_scale(q, P.d[j]) * (kt < nk ? 1.0f : 0.0f);
  };
  f32x16 acc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  bf16x8 B0_[2][4], B1[2][4];                  // decoded B of the current / next step

  // One K step k (position u = k % 4 in its super-step): reads x tile Ab,
  // multiplies with the decoded B `bo`, decodes the codes of step k+1 (read
  // here from the slab) with the block scales scales_next(j) into `bn`,
  // requests x tile k+3 into An, issues this step's scale loads
  // (issue_scales) and, at u == 2, the next super-step's code slab.
  auto step_k = [&](auto u_c, const u32x4* Ab, u32x4* An, const bf16x8 (&bo)[2][4], bf16x8 (&bn)[2][4],
                    auto&& issue_scales, auto&& scales_next, int64_t k) {
    constexpr int u = decltype(u_c)::value;
    u32x4 cw[2];
    read_codes(k + 1, cw);
    if constexpr (u == 2) {
      // the slab's last reads have landed: refill it first, so that waiting
      // for it (end of this step) leaves this step's x-tile and scale loads
      // in flight
      wait_lgkm0();
      asm volatile("" ::: "memory");
      dma_b(k / 4 + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    dma_a(imin(k + 3, nk - 1), An);
    __builtin_amdgcn_sched_barrier(0);
    issue_scales();
    __builtin_amdgcn_sched_barrier(0);
    MagTable tb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) tb[j] = make_table(cb, scales_next(j));
    // A fragments double-buffered across sub-steps: those of s+1 are read
    // while the MFMAs of s issue
    bf16x8 afr[2][8];
    auto read_frags = [&](int s, bf16x8 (&af)[8]) {
      const int sw = (4 * h + s) ^ a_swz(l32);     // a_swz(32 i + l32) == a_swz(l32)
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
        const uint32_t pw = s == 0 ? cw[j].x : s == 1 ? cw[j].y : s == 2 ? cw[j].z : cw[j].w;
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
  using U0 = std::integral_constant<int, 0>;
  using U1 = std::integral_constant<int, 1>;
  using U2 = std::integral_constant<int, 2>;
  using U3 = std::integral_constant<int, 3>;
  auto decode_step0 = [&](auto&& scale0) {
    u32x4 c0[2];
    read_codes(0, c0);
    bf16x8 (&bo)[2][4] = B0_;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const MagTable tb = make_table(cb, scale0(j));
      bo[j][0] = as_bf16x8(decode8(c0[j].x, tb));
      bo[j][1] = as_bf16x8(decode8(c0[j].y, tb));
      bo[j][2] = as_bf16x8(decode8(c0[j].z, tb));
      bo[j][3] = as_bf16x8(decode8(c0[j].w, tb));
    }
  };
  bf16x8 (&B0)[2][4] = B0_;
  auto nothing = [] {};

  // Prologue: the loads of "steps -2 and -1" in the order the loop issues
  // them, so that the loop's wait counts hold from step 0 on.
  // Vector-memory loads per step, in order: at u == 2 the code slab (8), then
  // x tile k+3 (8), then the scale loads (quad path: 4 at u == 1 for the next
  // super-step; per-step path: 4 for step k+2). The end of step k waits for x
  // tile k+1, issued in step k-2; whatever was issued after it may stay in
  // flight, and that count is the argument of each wait_vm below. Step u == 2
  // waits instead for the code slab it requested first (so only its own
  // x-tile and scale loads stay in flight): the next step reads that slab
  // right after the barrier. These explicit waits are what order the slab
  // DMA before its reads: the compiler's own LDS-DMA tracking cannot be
  // relied on to cover reads at other offsets of the slab.
  if constexpr (kQuad) {
    BScale4 Qc, Qn;
    load_s4(0, Qc);
    __builtin_amdgcn_sched_barrier(0);
    dma_a(0, As0);
    __builtin_amdgcn_sched_barrier(0);
    dma_b(0);
    __builtin_amdgcn_sched_barrier(0);
    dma_a(imin(1, nk - 1), As1);
    __builtin_amdgcn_sched_barrier(0);
    dma_a(imin(2, nk - 1), As2);
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<16>();                             // scales of super-step 0, x tile 0, code slab 0
    decode_step0([&](int j) { return scale_of(Qc, 0, 0, j); });
    lds_barrier();
    for (int64_t S = 0; S < nsup; ++S) {
      const int64_t k = 4 * S;
      step_k(U0{}, As0, As3, B0, B1, nothing, [&](int j) { return scale_of(Qc, 1, k + 1, j); }, k);
      wait_vm<16>();
      lds_barrier();
      step_k(U1{}, As1, As0, B1, B0, [&] { load_s4(S + 1, Qn); },
             [&](int j) { return scale_of(Qc, 2, k + 2, j); }, k + 1);
      wait_vm<20>();
      lds_barrier();
      step_k(U2{}, As2, As1, B0, B1, nothing, [&](int j) { return scale_of(Qc, 3, k + 3, j); }, k + 2);
      wait_vm<8>();                            // also the code slab requested first in this step
      lds_barrier();
      step_k(U3{}, As3, As2, B1, B0, nothing, [&](int j) { return scale_of(Qn, 0, k + 4, j); }, k + 3);
      wait_vm<28>();
      lds_barrier();
      Qc = Qn;
    }
  } else {
    BScale P0, P1;
    dma_a(0, As0);
    __builtin_amdgcn_sched_barrier(0);
    dma_b(0);
    __builtin_amdgcn_sched_barrier(0);
    dma_a(imin(1, nk - 1), As1);
    __builtin_amdgcn_sched_barrier(0);
    load_s(0, P0);
    __builtin_amdgcn_sched_barrier(0);
    dma_a(imin(2, nk - 1), As2);
    __builtin_amdgcn_sched_barrier(0);
    load_s(1, P1);
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<12>();                             // everything up to the scales of step 0
    // pin step 1's scales here: left alone, the (read-only) loads get sunk
    // into the loop entry, and the loop head would then drain every later load
    asm volatile("" ::"v"(static_cast<int>(P1.q[0])), "v"(static_cast<int>(P1.q[1])), "v"(P1.d[0]), "v"(P1.d[1]));
    decode_step0([&](int j) { return block_scale(P0.q[j], P0.d[j]) * P0.live; });
    lds_barrier();
    auto sc = [](const BScale& P, int j) { return block_scale(P.q[j], P.d[j]) * P.live; };
    for (int64_t S = 0; S < nsup; ++S) {
      const int64_t k = 4 * S;
      step_k(U0{}, As0, As3, B0, B1, [&] { load_s(k + 2, P0); }, [&](int j) { return sc(P1, j); }, k);
      wait_vm<28>();
      lds_barrier();
      step_k(U1{}, As1, As0, B1, B0, [&] { load_s(k + 3, P1); }, [&](int j) { return sc(P0, j); }, k + 1);
      wait_vm<28>();
      lds_barrier();
      step_k(U2{}, As2, As1, B0, B1, [&] { load_s(k + 4, P0); }, [&](int j) { return sc(P1, j); }, k + 2);
      wait_vm<12>();                           // also the code slab requested first in this step
      lds_barrier();
      step_k(U3{}, As3, As2, B1, B0, [&] { load_s(k + 5, P1); }, [&](int j) { return sc(P0, j); }, k + 3);
      wait_vm<36>();
      lds_barrier();
    }
  }
  wait_vm<0>();

  // epilogue: LoRA up-projection as a rank-r MFMA (RSN chunks of 16 ranks),
  // then bf16 stores
  if constexpr (RSN > 0) {
    const bool vec_ok = (r & 7) == 0;
    // All fragment loads of a group of row blocks go out before its MFMAs,
    // so their latency is paid once, not once per MFMA.
    auto lora = [&](auto rsn_c) {
      constexpr int RS = decltype(rsn_c)::value;
      constexpr int IG = RS <= 2 ? 8 : RS <= 4 ? 4 : 2;   // row blocks per group (registers)
      u32x4 bfr[2][RS];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t nrow = imin(n0 + 64 * w + 32 * j + l32, N - 1);
#pragma unroll
        for (int rs = 0; rs < RS; ++rs) bfr[j][rs] = load_row8(Bl + nrow * r, 16 * rs + 8 * h, r, vec_ok);
      }
#pragma unroll
      for (int i0 = 0; i0 < 8; i0 += IG) {
        u32x4 tf[IG][RS];
#pragma unroll
        for (int ii = 0; ii < IG; ++ii) {
          const int64_t mrow = imin(m0 + 32 * (i0 + ii) + l32, M - 1);
#pragma unroll
          for (int rs = 0; rs < RS; ++rs) tf[ii][rs] = ld16(tl + mrow * rp + 16 * rs + 8 * h);
        }
#pragma unroll
        for (int ii = 0; ii < IG; ++ii)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            f32x16 tmp;
#pragma unroll
            for (int v = 0; v < 16; ++v) tmp[v] = 0.f;
#pragma unroll
            for (int rs = 0; rs < RS; ++rs) tmp = mfma32(as_bf16x8(tf[ii][rs]), as_bf16x8(bfr[j][rs]), tmp);
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i0 + ii][j][v] += scale * tmp[v];
          }
      }
    };
    lora(std::integral_constant<int, RSN>{});
  }
  // bf16 stores: for fixed (i, j, v) the 32 lanes of a half-wave write 64
  // contiguous bytes of one row; interior tiles skip the bounds checks
  if (m0 + kTile <= M && n0 + kTile <= N) {
    uint16_t* yt = y + (m0 + 4 * h) * N + n0 + 64 * w + l32;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          yt[(32 * i + 8 * (v >> 2) + (v & 3)) * N + 32 * j] = bf16_bits(acc[i][j][v]);
  } else {
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
}

// ---------------------------------------------------------------------------
// k_gemm_bwd: dX [M, K] = dY . W' (+ LoRA), M > 16.
//
// Workgroup tile 256 (M) x 256 (K), eight waves (two per SIMD) as 2 x 4, each
// 128 x 64: 4 x 2 blocks of 32x32x16 bf16 MFMA. The contraction runs over W's
// rows (N) in steps of 64, so the weights are needed transposed: each step
// the workgroup decodes the 64 x 256 slice of W' (half a 64-block per thread,
// every weight once) into LDS, row-major, and the waves read their B operands
// with ds_read_b64_tr_b16. Two waves per SIMD let one wave's MFMAs issue
// while the other waits on its LDS reads, its decode or the step barrier.
// Per step k:
//   dY    tile k+1 (256 x 64) loaded into registers and written into the
//         other slot of a two-slot LDS ring at the end of the step (rows past
//         M read as zero);
//   codes of step k+2 loaded into registers (16 bytes per thread: eight
//         threads per weight row);
//   the MFMAs of step k run while the codes of step k+1 are decoded and
//         written into the other W' buffer.
// LDS: 2 x 32 KB (dY) + 2 x 36 KB (W', rows padded to 576 bytes so that a
// transposed read of 4 rows x 64 bytes covers all 64 banks once).
// ---------------------------------------------------------------------------
constexpr int kBwRow = 36;                     // 16-byte chunks per LDS row of the W' tile (32 + pad)
constexpr int kBwChunks = 64 * kBwRow;
constexpr int kBwThreads = 512;

struct BCodes {
  u32x4 p;         // this thread's 16 code bytes (half a 64-block)
  float d;
  int8_t q;
  float live;      // 1 for a real weight row, 0 past N
};

// RSN: rank chunks of 16 in the LoRA epilogue (1 for r <= 16, else rank_pad(r) / 16), 0 for none.
template <int RSN>
__global__ __launch_bounds__(kBwThreads, 1) void k_gemm_bwd(const uint16_t* __restrict__ dy, int64_t M, int64_t N,
                                                            int64_t K, const uint8_t* __restrict__ packed,
                                                            const int8_t* __restrict__ qscale,
                                                            const float* __restrict__ step,
                                                            const uint16_t* __restrict__ ul, int rp,
                                                            const uint16_t* __restrict__ Al, int r, float scale,
                                                            uint16_t* __restrict__ dx, Codebook cb) {
  // the two W' buffers are one array: after the main loop it holds A's
  // slice for the LoRA epilogue (up to 128 ranks x 256 columns)
  __shared__ u32x4 As0[kChunks];
  __shared__ u32x4 As1[kChunks];
  __shared__ u32x4 Ws[2 * kBwChunks];
  u32x4* const Ws0 = Ws;
  u32x4* const Ws1 = Ws + kBwChunks;
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = w >> 2, wn = w & 3;
  const int h = lane >> 5, l32 = lane & 31;
  const int ntm = static_cast<int>(cdiv(M, kTile)), ntk = static_cast<int>(cdiv(K, kTile));
  int tm, tk;
  tile_of(blockIdx.x, ntm, ntk, tm, tk);
  tm = __builtin_amdgcn_readfirstlane(tm);
  tk = __builtin_amdgcn_readfirstlane(tk);
  const int64_t m0 = static_cast<int64_t>(tm) * kTile, k0 = static_cast<int64_t>(tk) * kTile;
  const int64_t nbr = K / 64;
  const int64_t nsteps = cdiv(N, 64);

  // dY tile staging through registers (not LDS DMA: the transposed LDS reads
  // of W' carry no alias information, so any LDS DMA in flight would make the
  // compiler wait for it before each of them). Thread t moves 16-byte chunk
  // t & 7 of rows (t >> 3) + 64 i: eight lanes cover a row's 128 bytes.
  // Buffer loads through a descriptor over this tile's dY rows: rows past M
  // read as zero without a branch. (Columns past N in the last step read the
  // next row; the matching weight rows are dead, so they contribute zero.)
  const int ach = t & 7, arow0 = t >> 3;
  const int64_t rows_valid = imin(static_cast<int64_t>(kTile), M - m0);
  const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(dy + m0 * N), 0, static_cast<int>(rows_valid * N * 2), kBufferDword3);
  uint32_t aoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) aoff[i] = static_cast<uint32_t>((arow0 + 64 * i) * N * 2 + 16 * ach);
  u32x4 areg[4];
  auto load_a = [&](int64_t st) {
    const uint32_t so = static_cast<uint32_t>(imin(st, nsteps - 1) * 128);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      areg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(yr, aoff[i], so, 0));
  };
  auto store_a = [&](u32x4* Ab) {
#pragma unroll
    for (int i = 0; i < 4; ++i) Ab[a_slot(arow0 + 64 * i, ach)] = areg[i];
  };
  // this thread decodes half bh = t >> 8 (columns 32 bh .. 32 bh + 31) of
  // 64-column block t & 3 of weight row (t >> 2) & 63 of the step
  const int brow = (t >> 2) & 63, bkb = t & 3, bh = t >> 8;
  const int64_t bkbi = imin(k0 / 64 + bkb, nbr - 1);
  auto load_codes = [&](int64_t st, BCodes& P) {
    const int64_t n = st * 64 + brow;
    const int64_t nc = imin(n, N - 1);
    P.p = ld16(packed + nc * (K / 2) + bkbi * 32 + 16 * bh);
    const int64_t blk = nc * nbr + bkbi;
    P.q = qscale[blk];
    P.d = step[blk >> 8];
    P.live = n < N ? 1.0f : 0.0f;
  };
  // W' tile slot of (row, 16-byte chunk c of the 256 columns). Within each
  // 8-chunk block the chunk is xor-ed with the block index: a decode write
  // phase (4 rows x the 4 blocks, same chunk) then covers all 64 banks once,
  // and a transposed read phase (4 rows x 4 aligned chunks of one block) still does.
  auto w_slot = [](int row, int c) { return row * kBwRow + (c ^ ((c >> 3) & 3)); };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // B-operand reads (ds_read_b64_tr_b16): lane group G = lane / 16 reads rows
  // 16 s + 8 (G >> 1) + 4 q + (j16 >> 2), 4 columns at 4 (j16 & 3) of the
  // 16-column half (G & 1) of the wave's 32-column block j
  const int G = lane >> 4, j16 = lane & 15;
  const int hh = G >> 1, cbh = G & 1;
  auto read_bj = [&](const u32x4* Wb, int s, int j) {
    const int col = 64 * wn + 32 * j + 16 * cbh + 4 * (j16 & 3);
    s16x4 v[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int row = 16 * s + 8 * hh + 4 * q + (j16 >> 2);
      v[q] = ds_read_tr(Wb, w_slot(row, col >> 3) * 8 + (col & 4));
    }
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto read_b = [&](const u32x4* Wb, int s, bf16x8 (&bf)[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) bf[j] = read_bj(Wb, s, j);
  };
  auto read_a = [&](const u32x4* Ab, int s, bf16x8 (&af)[4]) {
    const int sw = (2 * s + h) ^ a_swz(l32);       // a_swz(128 wm + 32 i + l32) == a_swz(l32)
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = as_bf16x8(Ab[(128 * wm + 32 * i + l32) * 8 + sw]);
  };

  // one step: MFMAs on (Ab, Wb); decode `nx` into Wn; load dY tile st+1 and
  // write it into An in the last sub-step; load the codes of step st+2 into `ld`
  auto step_b = [&](const u32x4* Ab, u32x4* An, const u32x4* Wb, u32x4* Wn, const BCodes& nx, BCodes& ld,
                    int64_t st) {
    load_a(st + 1);
    __builtin_amdgcn_sched_barrier(0);
    load_codes(st + 2, ld);
    __builtin_amdgcn_sched_barrier(0);
    const MagTable tb = make_table(cb, block_scale(nx.q, nx.d) * nx.live);
    const uint32_t pw[4] = {nx.p.x, nx.p.y, nx.p.z, nx.p.w};
    bf16x8 af[2][4], bf[2][2];
    read_a(Ab, 0, af[0]);
    read_b(Wb, 0, bf[0]);
    __builtin_amdgcn_sched_barrier(0);
    // Each sub-step is its own scheduling region, issued in this order: its
    // first MFMA (operands read during the previous sub-step), then per MFMA
    // one fragment read of the next sub-step and a share of the decode, then
    // its W' write (and in the last one the dY writes).
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) {
        read_a(Ab, s + 1, af[(s + 1) & 1]);
        read_b(Wb, s + 1, bf[(s + 1) & 1]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[s & 1][i], bf[s & 1][j], acc[i][j]);
      Wn[w_slot(brow, 8 * bkb + 4 * bh + s)] = decode8(pw[s], tb);
      if (s == 3) store_a(An);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (s < 3) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
      }
      if (s == 3)
        __builtin_amdgcn_sched_group_barrier(0x200, 5, 0);
      else
        __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // prologue: dY tile 0, codes of steps 0 and 1; decode step 0
  BCodes P0, P1;
  load_a(0);
  __builtin_amdgcn_sched_barrier(0);
  load_codes(0, P0);
  __builtin_amdgcn_sched_barrier(0);
  load_codes(1, P1);
  __builtin_amdgcn_sched_barrier(0);
  store_a(As0);
  asm volatile("" ::"v"(P1.p), "v"(static_cast<int>(P1.q)), "v"(P1.d));
  {
    const MagTable tb = make_table(cb, block_scale(P0.q, P0.d) * P0.live);
    const uint32_t pw[4] = {P0.p.x, P0.p.y, P0.p.z, P0.p.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) Ws0[w_slot(brow, 8 * bkb + 4 * bh + c)] = decode8(pw[c], tb);
  }
  __syncthreads();
  // The end of step st waits for this wave's LDS writes (W' and dY of step
  // st+1), then the barrier publishes them; the code loads of step st+2 stay
  // in flight.
  for (int64_t st = 0; st < nsteps; st += 2) {
    step_b(As0, As1, Ws0, Ws1, P1, P0, st);
    __builtin_amdgcn_s_waitcnt(0xC07F);        // lgkmcnt(0)
    lds_barrier();
    step_b(As1, As0, Ws1, Ws0, P0, P1, st + 1);
    __builtin_amdgcn_s_waitcnt(0xC07F);
    lds_barrier();
  }
  wait_vm<0>();

  if constexpr (RSN > 0) {
    // The up-projection contracts over the ranks: its B operand is the r x 256
    // slice of A under this tile, staged row-major in the W' buffers (free
    // after the main loop; the same padded, swizzled rows) and read with the
    // main loop's transposed reads, rank chunk rs in place of sub-step s.
    // Ranks past r and columns past K are zero. RSN counts the rank chunks
    // of 16 that are used (1 for r <= 16: u's padding columns 16 .. 31 are
    // zero and skipped).
    static_assert(16 * 8 * kBwRow <= 2 * kBwChunks, "A's slice does not fit the W' buffers");
    __syncthreads();
    {
      // 16 RSN rows x 32 chunks of 8 columns (K % 64 == 0, so a chunk is
      // wholly inside or past K), all loads before the LDS writes
      constexpr int kPer = 16 * RSN * 32 / kBwThreads;
      u32x4 av[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int e = t + kBwThreads * u, j = e >> 5, ch = e & 31;
        const int64_t kc = k0 + 8 * ch;
        av[u] = (j < r && kc < K) ? ld16(Al + static_cast<int64_t>(j) * K + kc) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int e = t + kBwThreads * u;
        Ws[w_slot(e >> 5, e & 31)] = av[u];
      }
    }
    __syncthreads();
    // groups of IG row blocks: their u fragments are loaded before their
    // MFMAs; A's fragments read per column block
    auto lora = [&](auto rsn_c) {
      constexpr int RS = decltype(rsn_c)::value;
      constexpr int IG = RS <= 2 ? 4 : RS <= 4 ? 2 : 1;
#pragma unroll
      for (int i0 = 0; i0 < 4; i0 += IG) {
        u32x4 uf[IG][RS];
#pragma unroll
        for (int ii = 0; ii < IG; ++ii) {
          const int64_t mrow = imin(m0 + 128 * wm + 32 * (i0 + ii) + l32, M - 1);
#pragma unroll
          for (int rs = 0; rs < RS; ++rs) uf[ii][rs] = ld16(ul + mrow * rp + 16 * rs + 8 * h);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          bf16x8 bl[RS];
#pragma unroll
          for (int rs = 0; rs < RS; ++rs) bl[rs] = read_bj(Ws, rs, j);
#pragma unroll
          for (int ii = 0; ii < IG; ++ii) {
            f32x16 tmp;
#pragma unroll
            for (int v = 0; v < 16; ++v) tmp[v] = 0.f;
#pragma unroll
            for (int rs = 0; rs < RS; ++rs) tmp = mfma32(as_bf16x8(uf[ii][rs]), bl[rs], tmp);
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i0 + ii][j][v] += scale * tmp[v];
          }
        }
      }
    };
    lora(std::integral_constant<int, RSN>{});
  }
  if (m0 + kTile <= M && k0 + kTile <= K) {
    uint16_t* dt = dx + (m0 + 128 * wm + 4 * h) * K + k0 + 64 * wn + l32;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          dt[(32 * i + 8 * (v >> 2) + (v & 3)) * K + 32 * j] = bf16_bits(acc[i][j][v]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t kk = k0 + 64 * wn + 32 * j + l32;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t mm = m0 + 128 * wm + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
          if (mm < M && kk < K) dx[mm * K + kk] = bf16_bits(acc[i][j][v]);
        }
      }
  }
}

// ---------------------------------------------------------------------------
// dispatch: LoRA down-projection, then the small-M or the tiled kernel
// ---------------------------------------------------------------------------
// The tiled forward over a table of up to kFwdMaxWeights weights at one M:
// the LoRA down-projection of each weight into its own workspace slice (one
// launch each), then one launch of k_gemm_fwd for all of them. Weight i's
// workspace is ws + i * ws_stride (its layout ws_layout(0, M, N[i], K[i], r)).
static hipError_t launch_fwd_tiled(int64_t M, int G, const uint16_t* const* x, const int64_t* N, const int64_t* K,
                                   const uint8_t* const* packed, const int8_t* const* qscale,
                                   const float* const* step, const uint16_t* const* A, const uint16_t* const* B,
                                   int r, float alpha, uint16_t* const* y, void* ws, size_t ws_stride,
                                   const Codebook& cb, hipStream_t stream) {
  const float scale = r > 0 ? alpha / static_cast<float>(r) : 0.0f;
  const int rp = r > 0 ? static_cast<int>(rank_pad(r)) : 0;
  FwdTable tab{};
  tab.count = G;
  bool quad = true;
  int cols = 0;
  for (int i = 0; i < G; ++i) {
    const WsLayout L = ws_layout(0, M, N[i], K[i], r);
    char* wsb = static_cast<char*>(ws) + static_cast<size_t>(i) * ws_stride;
    void* lora = r > 0 ? static_cast<void*>(wsb + L.lora_off) : nullptr;
    if (r > 0) {
      const hipError_t e = launch_lora_down(true, x[i], M, K[i], A[i], r, lora, stream, nullptr,
                                            reinterpret_cast<float*>(wsb + L.dp_off));
      if (e != hipSuccess) return e;
    }
    tab.x[i] = x[i];
    tab.packed[i] = packed[i];
    tab.qscale[i] = qscale[i];
    tab.step[i] = step[i];
    tab.tl[i] = static_cast<const uint16_t*>(lora);
    tab.B[i] = r > 0 ? B[i] : nullptr;
    tab.y[i] = y[i];
    tab.N[i] = static_cast<int>(N[i]);
    tab.K[i] = static_cast<int>(K[i]);
    tab.col0[i] = cols;
    cols += static_cast<int>(cdiv(N[i], kTile));
    quad = quad && K[i] % 256 == 0;
  }
  tab.col0[G] = cols;
  const int64_t tiles = cdiv(M, kTile) * cols;
#define QNF4_FWD(RSNV)                                                                                          \
  do {                                                                                                         \
    if (quad)                                                                                                  \
      hipLaunchKernelGGL(HIP_KERNEL_NAME(k_gemm_fwd<true, RSNV>), dim3(static_cast<unsigned>(tiles)), dim3(256), \
                         0, stream, tab, M, rp, r, scale, cb);                                                 \
    else                                                                                                       \
      hipLaunchKernelGGL(HIP_KERNEL_NAME(k_gemm_fwd<false, RSNV>), dim3(static_cast<unsigned>(tiles)),          \
                         dim3(256), 0, stream, tab, M, rp, r, scale, cb);                                      \
  } while (0)
  mark_kernel(0, stream);
  switch (r == 0 ? 0 : r <= 16 ? 1 : rp / 16) {
    case 0: QNF4_FWD(0); break;
    case 1: QNF4_FWD(1); break;
    case 2: QNF4_FWD(2); break;
    case 4: QNF4_FWD(4); break;
    case 6: QNF4_FWD(6); break;
    default: QNF4_FWD(8); break;
  }
#undef QNF4_FWD
  mark_kernel(1, stream);
  return hipGetLastError();
}

hipError_t launch_lora_fwd(const uint16_t* x, int64_t M, int64_t N, int64_t K, const uint8_t* packed,
                           const int8_t* qscale, const float* step, const uint16_t* A, const uint16_t* B,
                           int r, float alpha, uint16_t* y, void* ws, const Codebook& cb,
                           hipStream_t stream) {
  if (M <= kSmallM)
    return launch_dec_fwd(M, 1, &x, &N, &K, &packed, &qscale, &step, &A, &B, r, alpha, &y, ws, cb, stream);
  return launch_fwd_tiled(M, 1, &x, &N, &K, &packed, &qscale, &step, &A, &B, r, alpha, &y, ws, 0, cb, stream);
}

// Tiled batches go in chunks of kFwdMaxWeights, each weight with a workspace
// slice of the largest single-weight size in the batch.
static size_t tiled_stride(int64_t M, int G, const int64_t* N, const int64_t* K, int r) {
  size_t need = 0;
  for (int i = 0; i < G; ++i) {
    const size_t b = align256(ws_layout(0, M, N[i], K[i], r).total);
    need = b > need ? b : need;
  }
  return need;
}

size_t batched_ws_bytes(int64_t M, int G, const int64_t* N, const int64_t* K, int r) {
  if (M <= kSmallM) return dec_workspace_bytes(M, G, N, K);
  const int per_launch = G < kFwdMaxWeights ? G : kFwdMaxWeights;
  return tiled_stride(M, G, N, K, r) * static_cast<size_t>(per_launch);
}

hipError_t launch_lora_fwd_batched(int64_t M, int G, const uint16_t* const* x, const int64_t* N, const int64_t* K,
                                   const uint8_t* const* packed, const int8_t* const* qscale,
                                   const float* const* step, const uint16_t* const* A, const uint16_t* const* B,
                                   int r, float alpha, uint16_t* const* y, void* ws, const Codebook& cb,
                                   hipStream_t stream) {
  if (M <= kSmallM) return launch_dec_fwd(M, G, x, N, K, packed, qscale, step, A, B, r, alpha, y, ws, cb, stream);
  const size_t stride = tiled_stride(M, G, N, K, r);
  for (int c0 = 0; c0 < G; c0 += kFwdMaxWeights) {
    const int cn = G - c0 < kFwdMaxWeights ? G - c0 : kFwdMaxWeights;
    const hipError_t e = launch_fwd_tiled(M, cn, x + c0, N + c0, K + c0, packed + c0, qscale + c0, step + c0,
                                          r ? A + c0 : nullptr, r ? B + c0 : nullptr, r, alpha, y + c0, ws, stride,
                                          cb, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_bwd_dx(const uint16_t* dy, int64_t M, int64_t N, int64_t K, const uint8_t* packed,
                         const int8_t* qscale, const float* step, const uint16_t* A, const uint16_t* B,
                         int r, float alpha, uint16_t* dx, void* ws, const Codebook& cb,
                         hipStream_t stream) {
  // small M: the down-projection u = dY . B is computed inside k_dec_bwd
  if (M <= kSmallM)
    return launch_dec_bwd(M, 1, &dy, &N, &K, &packed, &qscale, &step, &A, &B, r, alpha, &dx, ws, cb, stream);
  const WsLayout L = ws_layout(1, M, N, K, r);
  char* wsb = static_cast<char*>(ws);
  const float scale = r > 0 ? alpha / static_cast<float>(r) : 0.0f;
  const int rp = r > 0 ? static_cast<int>(rank_pad(r)) : 0;
  void* lora = r > 0 ? static_cast<void*>(wsb + L.lora_off) : nullptr;
  if (r > 0) {
    const hipError_t e = launch_lora_down(false, dy, M, N, B, r, lora, stream,
                                          reinterpret_cast<uint16_t*>(wsb + L.bt_off),
                                          reinterpret_cast<float*>(wsb + L.dp_off));
    if (e != hipSuccess) return e;
  }
  const int64_t tiles = cdiv(M, kTile) * cdiv(K, kTile);
#define QNF4_BWD(RSNV)                                                                                         \
  hipLaunchKernelGGL(HIP_KERNEL_NAME(k_gemm_bwd<RSNV>), dim3(static_cast<unsigned>(tiles)), dim3(kBwThreads), 0, \
                     stream,                                                                                  \
                     dy, M, N, K, packed, qscale, step, static_cast<const uint16_t*>(lora), rp, A, r, scale, dx, cb)
  mark_kernel(0, stream);
  switch (r == 0 ? 0 : r <= 16 ? 1 : rp / 16) {
    case 0: QNF4_BWD(0); break;
    case 1: QNF4_BWD(1); break;
    case 2: QNF4_BWD(2); break;
    case 4: QNF4_BWD(4); break;
    case 6: QNF4_BWD(6); break;
    default: QNF4_BWD(8); break;
  }
#undef QNF4_BWD
  mark_kernel(1, stream);
  return hipGetLastError();
}

size_t bwd_batched_ws_bytes(int64_t M, int G, const int64_t* N, const int64_t* K, int r) {
  if (M <= kSmallM) return dec_bwd_workspace_bytes(M, G, N, K);
  size_t most = 0;                           // the tiled calls run one after another on one workspace
  for (int i = 0; i < G; ++i) {
    const size_t b = ws_layout(1, M, N[i], K[i], r).total;
    if (b > most) most = b;
  }
  return most;
}

hipError_t launch_bwd_dx_batched(int64_t M, int G, const uint16_t* const* dy, const int64_t* N, const int64_t* K,
                                 const uint8_t* const* packed, const int8_t* const* qscale,
                                 const float* const* step, const uint16_t* const* A, const uint16_t* const* B,
                                 int r, float alpha, uint16_t* const* dx, void* ws, const Codebook& cb,
                                 hipStream_t stream) {
  if (M <= kSmallM) return launch_dec_bwd(M, G, dy, N, K, packed, qscale, step, A, B, r, alpha, dx, ws, cb, stream);
  for (int i = 0; i < G; ++i) {
    const hipError_t e = launch_bwd_dx(dy[i], M, N[i], K[i], packed[i], qscale[i], step[i], r ? A[i] : nullptr,
                                       r ? B[i] : nullptr, r, alpha, dx[i], ws, cb, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace qnf4
