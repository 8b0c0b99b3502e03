// Decode-shaped (M <= 16) fused NF4-dequant forward for gfx950, over a table
// of weights in one launch.
//
//   y_p = bf16( x_p . W_p'^T + (alpha/r) . (x_p . A_p^T) . B_p^T )
//
// for every weight p of the table ("A 65B fine-tune on the GPU you already
// have", figure 2: the weights become bf16 block by block right before the
// multiply; "QLoRA and Quantized Training", "In code": r and lora_alpha). At
// these shapes each weight is used by at most 16 rows, so the kernel is bound
// by streaming the 0.516 bytes/param stored weight from HBM and by the VALU
// work of decoding it; it is written for both.
//
// Work items. An item is 256 weight rows x a range of K of one weight, run by
// one workgroup of four waves (64 rows each, four 16-row MFMA tiles). A
// weight's K is split into S ranges when the launch has too few row blocks to
// fill the chip; every split writes fp32 partial sums and the last split of a
// row block to arrive (an arrival counter in the workspace) adds them in split
// order, so results do not depend on scheduling. Items of one row block run on
// one XCD (consecutive workgroup ids go round robin over the 8 XCDs, and items
// are assigned so that each XCD gets a contiguous range), so their partials and
// the shared x and adapter lines stay in that XCD's L2.
//
// Main loop, per 256-deep super-step: lane (g, c) of a wave holds block
// 4 ss + g of weight row c of each of its four tiles (32 code bytes = the
// B operands of eight 16x16x32 MFMAs) and the matching 64 activations of row c
// of x (the A operands). The next super-step's codes, scales and activations
// are loaded while the current one is decoded and multiplied.
//
// LoRA. Each item computes t = x . A^T over its own K range (wave w takes the
// super-steps ss with ss % 4 == w, from the same activation fragments), the
// four waves' parts are summed through LDS, and t . B^T is added to the item's
// partial sums with t carried as the sum of two bf16 values (hi + lo, about 16
// significant bits), so splitting K leaves the LoRA term exact to fp32-level
// rounding instead of requiring the full-K t before any output.
//
// Decode. A block's 64 weights share one scale s, so they take at most 16
// values; the levels are exactly antisymmetric, so the 8 magnitudes
// |bf16(L[c] s)| (c < 8, largest first) and a sign give all 16. Code c maps to
// magnitude index c (c < 8) or 15 - c (c >= 8), which is c XOR 7b with b = bit 3
// of c, masked to 3 bits; all eight nibbles of a packed word are transformed at
// once. The two bf16 byte planes are looked up with v_perm_b32, the sign
// (c < 8) is OR-ed into the high bytes, and the even and odd elements are paired
// without interleaving: the word decodes to the element order
// 0 2 4 6 1 3 5 7, and the activation fragments are permuted the same way
// (a contraction does not depend on the order of its terms). 17 VALU
// operations per 8 weights.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "mm_common.hpp"

namespace qnf4 {

constexpr int kDecNT = 4;                         // 16-row MFMA tiles per wave
constexpr int kDecBufWord3 = 0x00020000;          // raw buffer descriptor word 3 on gfx9-family parts
constexpr int kDecRows = 16 * kDecNT * 4;         // weight rows per item (four waves)
constexpr int64_t kDecMaxSps = 8;               // 256-deep super-steps per item at most
constexpr int kDecEarlyBItems = 768;            // launches up to this many items request B early

__device__ __forceinline__ int dec_item_of(int wg, int grid) {
  // grid is a multiple of 8: XCD (wg % 8) gets items [xcd * grid/8, ...)
  return (wg & 7) * (grid >> 3) + (wg >> 3);
}

// LDS staging of one 256-deep super-step, shared by the workgroup's four waves:
// 16 rows of x (rows past M zero) and, for ranks up to 16, the 16 adapter
// rows, each row 32 chunks of 16 bytes with chunk k of row q at position
// k ^ (q & 15) -- the 16 lanes of a read phase (rows c = 0..15, one logical
// chunk) then touch 16 distinct bank groups.
constexpr int kDecStageChunks = 2 * 16 * 32;      // x part, then adapter part
__device__ __forceinline__ int dec_slot(int row, int chunk) { return row * 32 + (chunk ^ (row & 15)); }

// RT: rank tiles of 16 the kernel computes (0: no adapter; else a power of two
// with 16 RT >= r). kQuad: every K of the launch is a multiple of 256.
template <int RT, bool kQuad>
__global__ __launch_bounds__(256, 2) void k_dec_fwd(DecFwdBatch bt, Codebook cb) {
  constexpr int kRT = RT > 0 ? RT : 1;
  constexpr int kRS = RT > 1 ? RT / 2 : 1;      // 32-deep rank chunks of the up-projection
  constexpr bool kStageA = RT == 1;             // adapter rows staged in LDS with x
  // two stages of x (+ adapter), and for kQuad the item's scale codes and
  // steps per (row, super-step); after the main loop the same memory holds
  // the four waves' parts of t
  __shared__ u32x4 stg0[kDecStageChunks], stg1[kDecStageChunks];
  __shared__ uint32_t lq[kQuad ? kDecRows * kDecMaxSps : 1];
  __shared__ float ld[kQuad ? kDecRows * kDecMaxSps : 1];
  __shared__ int last_flag;
  float* const tsh = reinterpret_cast<float*>(stg0);

  // workgroup barrier that orders the compiler's LDS accesses too
  auto sync = [&] { lds_barrier_on(stg0, stg1, lq, ld); };

  const int item = dec_item_of(blockIdx.x, gridDim.x);
  if (item >= bt.items) return;
  int pi = 0;
#pragma unroll
  for (int i = 1; i < kDecMaxProblems; ++i)
    if (i < bt.count && item >= bt.p[i].item0) pi = i;
  const DecFwdProblem& P = bt.p[pi];

  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int M = bt.M, r = bt.r;
  // sizes fit 32 bits (N, K <= 2^21): only the base addresses are 64-bit
  const int N = P.N, K = P.K;
  const int nbr = K / 64, nss = (nbr + 3) / 4;
  const int local = item - P.item0;
  const int b = local / P.S, s = local - (local / P.S) * P.S;
  const int ss0 = s * P.sps;
  const int ss1 = ss0 + P.sps < nss ? ss0 + P.sps : nss;
  const int nit = ss1 - ss0;
  const int nb0 = b * kDecRows + 64 * w;                 // this wave's first row

  // Every operand is read through a buffer descriptor whose range check
  // returns zero outside it: the wave's 64 weight rows, their scale codes and
  // steps (rows past N read as zero codes with a zero scale), x (rows past M),
  // the adapter (rows past r). Values that are wave-uniform by construction go
  // through readfirstlane so that the descriptors live in scalar registers.
  const int rows_valid = __builtin_amdgcn_readfirstlane(N - nb0 < 0 ? 0 : (N - nb0 < 64 ? N - nb0 : 64));
  const int nbw = __builtin_amdgcn_readfirstlane(nb0 < N ? nb0 : 0);
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(P.packed + static_cast<int64_t>(nbw) * (K / 2)), 0, rows_valid * (K / 2), kDecBufWord3);
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(P.x), 0, M * K * 2, kDecBufWord3);
  const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(RT > 0 ? P.A : P.x), 0, RT > 0 ? r * K * 2 : 0, kDecBufWord3);

  // The super-steps of the item in an order rotated per workgroup, so that
  // the workgroups resident at one time read different 128-byte columns of
  // their rows (the sum over K does not depend on the order).
  const int rot = nit > 0 ? (b * 5) % nit : 0;
  auto ss_of = [&](int i) {
    const int j = i + rot;
    return ss0 + (j >= nit ? j - nit : j);
  };

  // scale codes and steps of this lane's rows (kQuad: one aligned word of four
  // codes and one step per row and super-step, kept in LDS for the item; else
  // loaded with the codes)
  const int64_t blk0w = static_cast<int64_t>(nbw) * nbr;
  const int sb0w = __builtin_amdgcn_readfirstlane(static_cast<int>(blk0w & 255));
  const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(P.qscale + blk0w), 0, rows_valid * nbr, kDecBufWord3);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(P.step + (blk0w >> 8)), 0, ((sb0w + rows_valid * nbr + 255) >> 8) * 4, kDecBufWord3);
  // stage DMA: wave w moves chunks [256 w, 256 w + 256) of the stage, four
  // instructions of 64 lanes; lane l of instruction h lands at slot
  // 256 w + 64 h + l, i.e. row q = slot / 32 (x rows 0-15, then adapter rows),
  // physical chunk slot % 32, and fetches logical chunk phys ^ (q & 15)
  uint32_t doff[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int slot = 256 * w + 64 * h + lane;
    const int q = (slot >> 5) & 15, phys = slot & 31;
    doff[h] = static_cast<uint32_t>(q * K * 2 + ((phys ^ q) * 16));
  }
  auto dma_stage = [&](int ss, u32x4* stg) {
    const uint32_t so = static_cast<uint32_t>(ss * 512);
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      lds_void* dst = (lds_void*)(stg + 256 * w + 64 * h);
      if (w < 2)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, dst, 16, doff[h], so, 0, 0);
      else if (kStageA)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, dst, 16, doff[h], so, 0, 0);
    }
  };
  // wave-uniform number of stage-DMA instructions this wave issues
  const int ndma = (w < 2 || kStageA) ? 4 : 0;

  f32x4 acc[kDecNT], tacc[kRT];
#pragma unroll
  for (int nt = 0; nt < kDecNT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int jt = 0; jt < kRT; ++jt) tacc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // codes (and for ragged K the scale codes and steps) of super-step ss,
  // requested one super-step ahead into registers
  struct Codes {
    u32x4 cw[kDecNT][2];
    float d[kQuad ? 1 : kDecNT];
    uint32_t q[kQuad ? 1 : kDecNT];
  };
  auto load_codes = [&](int ss, Codes& C) {
    const int kbr = ss * 4 + g;
    const int kb = kbr < nbr ? kbr : nbr - 1;
#pragma unroll
    for (int nt = 0; nt < kDecNT; ++nt) {
      const int row = 16 * nt + c;
      const uint32_t co = static_cast<uint32_t>(row * (K / 2) + kb * 32);
      C.cw[nt][0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(crs, co, 0, 0));
      C.cw[nt][1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(crs, co + 16, 0, 0));
      if constexpr (!kQuad) {
        const int bl = row * nbr + kb;
        C.q[nt] = __builtin_amdgcn_raw_buffer_load_b8(qrs, static_cast<uint32_t>(bl), 0, 0);
        C.d[nt] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(srs, static_cast<uint32_t>(((sb0w + bl) >> 8) * 4), 0, 0));
      }
    }
  };
  // adapter rows 16 jt + c of block kb, pieces 2w and 2w + 1, straight from
  // memory (ranks past 16; lanes past K read zero)
  auto load_adapter = [&](int ss, int jt, u32x4 (&a)[2]) {
    const int kbr = ss * 4 + g;
    const int kb = kbr < nbr ? kbr : nbr - 1;
    const uint32_t o = static_cast<uint32_t>(((16 * jt + c) * K + kb * 64 + 16 * w) * 2);
    const uint32_t off = kbr < nbr ? o : 0x80000000u;
    a[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ars, off, 0, 0));
    a[1] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ars, off + 16, 0, 0));
  };

  Codes c0, c1;
  if constexpr (kQuad) {
    // thread t owns row 64 w + lane of the workgroup's 256 rows
    uint32_t qv[kDecMaxSps];
    float dv[kDecMaxSps];
#pragma unroll
    for (int u = 0; u < kDecMaxSps; ++u) {
      const int bl = lane * nbr + (ss0 + u) * 4;
      const bool in = u < nit;
      qv[u] = in ? __builtin_amdgcn_raw_buffer_load_b32(qrs, static_cast<uint32_t>(bl), 0, 0) : 0u;
      dv[u] = in ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                       srs, static_cast<uint32_t>(((sb0w + bl) >> 8) * 4), 0, 0))
                 : 0.0f;
    }
    __builtin_amdgcn_sched_barrier(0);
    if (nit > 0) {                                 // the first stage goes out behind them
      load_codes(ss_of(0), c0);
      dma_stage(ss_of(0), stg0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kDecMaxSps; ++u) {
      lq[t * kDecMaxSps + u] = qv[u];
      ld[t * kDecMaxSps + u] = dv[u];
    }
    sync();
  } else if (nit > 0) {
    load_codes(ss_of(0), c0);
    dma_stage(ss_of(0), stg0);
  }


  // B rows of the LoRA up-projection for this lane's four weight rows. In
  // launches of at most one round of workgroups (a single weight or a small
  // group: the workgroup's one item is the whole of its time) and with
  // 16-byte rows (r % 8 == 0) they are requested at the start of the last
  // super-step, so their latency overlaps its decode instead of adding one
  // more round trip after it; in larger launches other items cover that
  // latency and the registers are better left to the main loop. Pieces past r
  // read as zero (out-of-range offset); rows past N repeat the last row (their
  // outputs are never written).
  constexpr int kRSb = RT > 0 ? kRS : 1;
  u32x4 bop[kDecNT][kRSb];
  const bool early_b = RT > 0 && (r & 7) == 0 && bt.items <= kDecEarlyBItems;
  const __amdgpu_buffer_rsrc_t bbr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(RT > 0 ? P.B : P.x), 0, RT > 0 ? N * r * 2 : 0, kDecBufWord3);
  auto load_b_early = [&] {
#pragma unroll
    for (int nt = 0; nt < kDecNT; ++nt) {
      const int n = nb0 + 16 * nt + c < N ? nb0 + 16 * nt + c : N - 1;
#pragma unroll
      for (int rs = 0; rs < kRSb; ++rs) {
        const int col = 32 * rs + 8 * g;
        const uint32_t off = col < r ? static_cast<uint32_t>((n * r + col) * 2) : 0x80000000u;
        bop[nt][rs] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(bbr, off, 0, 0));
      }
    }
  };

  // iteration i: (1) every wave is past its reads of the stage buffer about to
  // be refilled (barrier); (2) request the codes and the stage of the next
  // super-step; (3) wait until this wave's part of the current stage has
  // landed, then for all waves' parts (barrier); (4) decode and multiply.
  // The waits are explicit: the compiler does not track LDS written by DMA.
  auto iter = [&](auto pre, int i, const Codes& cur, Codes& nxt, const u32x4* stg, u32x4* stg_next) {
    constexpr bool kPre = decltype(pre)::value;
    const int ss = ss_of(i);
    // the lane's k-block is past K only in the ragged last super-step
    const bool kvalid = kQuad || ss * 4 + g < nbr;
    const uint32_t lv = kvalid ? 0xFFFFFFFFu : 0u;
    const u32x4 live = {lv, lv, lv, lv};
    sync();
    if constexpr (kPre) {
      load_codes(ss_of(i + 1), nxt);
      dma_stage(ss_of(i + 1), stg_next);
      __builtin_amdgcn_sched_barrier(0);
      // outstanding, oldest first: [codes i, stage i] [codes i+1, stage i+1]
      if (ndma) wait_vm<2 * kDecNT + 4 + (kQuad ? 0 : 2 * kDecNT)>();
      else wait_vm<2 * kDecNT + (kQuad ? 0 : 2 * kDecNT)>();
    } else if (RT > 0 && early_b) {
      load_b_early();
      __builtin_amdgcn_sched_barrier(0);
      wait_vm<kDecNT * kRSb>();                  // codes and stage of this step, not B
    } else {
      wait_vm<0>();
    }
    sync();
    // past K the staged rows hold the next row's values: the lane's
    // activations (and adapter values) are masked to zero there
    u32x4 xa[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) xa[j] = perm8(stg[dec_slot(c, 8 * g + j)]) & live;
#pragma unroll
    for (int nt = 0; nt < kDecNT; ++nt) {
      float sc;
      if constexpr (kQuad) {
        const int row = 64 * w + 16 * nt + c;
        const int8_t qc = static_cast<int8_t>(lq[row * kDecMaxSps + (ss - ss0)] >> (8 * g));
        sc = block_scale(qc, ld[row * kDecMaxSps + (ss - ss0)]);
      } else {
        sc = kvalid ? block_scale(static_cast<int8_t>(cur.q[nt]), cur.d[nt]) : 0.0f;
      }
      const MagTable tb = make_table(cb, sc);
      const uint32_t pw[8] = {cur.cw[nt][0].x, cur.cw[nt][0].y, cur.cw[nt][0].z, cur.cw[nt][0].w,
                              cur.cw[nt][1].x, cur.cw[nt][1].y, cur.cw[nt][1].z, cur.cw[nt][1].w};
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[nt] = mfma16(as_bf16x8(xa[j]), as_bf16x8(decode8_perm(pw[j], tb)), acc[nt]);
    }
    if constexpr (RT > 0) {
      // pieces 2w, 2w + 1 of the lane's 64 activations (wave-uniform index)
      const u32x4 x0 = w == 0 ? xa[0] : w == 1 ? xa[2] : w == 2 ? xa[4] : xa[6];
      const u32x4 x1 = w == 0 ? xa[1] : w == 1 ? xa[3] : w == 2 ? xa[5] : xa[7];
      if constexpr (kStageA) {
        const u32x4 a0 = stg[16 * 32 + dec_slot(c, 8 * g + 2 * w)] & live;
        const u32x4 a1 = stg[16 * 32 + dec_slot(c, 8 * g + 2 * w + 1)] & live;
        tacc[0] = mfma16(as_bf16x8(x0), as_bf16x8(perm8(a0)), tacc[0]);
        tacc[0] = mfma16(as_bf16x8(x1), as_bf16x8(perm8(a1)), tacc[0]);
      } else {
#pragma unroll
        for (int jt = 0; jt < kRT; ++jt) {
          u32x4 a[2];
          load_adapter(ss, jt, a);
          tacc[jt] = mfma16(as_bf16x8(x0), as_bf16x8(perm8(a[0])), tacc[jt]);
          tacc[jt] = mfma16(as_bf16x8(x1), as_bf16x8(perm8(a[1])), tacc[jt]);
        }
      }
    }
  };

  using Pre = std::integral_constant<bool, true>;
  using NoPre = std::integral_constant<bool, false>;
  int i = 0;
  for (; i + 2 < nit; i += 2) {
    iter(Pre{}, i, c0, c1, stg0, stg1);
    iter(Pre{}, i + 1, c1, c0, stg1, stg0);
  }
  if (i + 1 < nit) {
    iter(Pre{}, i, c0, c1, stg0, stg1);
    iter(NoPre{}, i + 1, c1, c0, stg1, stg0);
  } else if (i < nit) {
    iter(NoPre{}, i, c0, c1, stg0, stg1);
  }
  sync();                                  // the stage buffers become the t exchange

  // LoRA: sum the four waves' parts of t (fixed order), then add
  // scale * (t_hi + t_lo) . B^T to each tile
  if (RT > 0) {
    // rows padded against bank conflicts where the 64 rows still fit in the stage buffers
    constexpr int kLd = 16 * kRT + (kRT < 8 ? 4 : 0);
    static_assert(4 * 16 * kLd * 4 <= sizeof(u32x4) * 2 * kDecStageChunks, "t exchange exceeds the stage buffers");
    if (!early_b || nit == 0) {
#pragma unroll
      for (int nt = 0; nt < kDecNT; ++nt) {
        const int64_t n = imin(nb0 + 16 * nt + c, N - 1);
#pragma unroll
        for (int rs = 0; rs < kRS; ++rs)
          bop[nt][rs] = load_row8(P.B + n * r, 32 * rs + 8 * g, r, (r & 7) == 0);
      }
    }
#pragma unroll
    for (int jt = 0; jt < kRT; ++jt)
#pragma unroll
      for (int v = 0; v < 4; ++v) tsh[(w * 16 + 4 * g + v) * kLd + 16 * jt + c] = tacc[jt][v];
    __syncthreads();
#pragma unroll
    for (int rs = 0; rs < kRS; ++rs) {
      float tv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = 32 * rs + 8 * g + e;
        float sum = 0.f;
        if (j < 16 * kRT) {
#pragma unroll
          for (int ww = 0; ww < 4; ++ww) sum += tsh[(ww * 16 + c) * kLd + j];
        }
        tv[e] = sum;
      }
      u32x4 hi, lo;
      hi.x = pack_bf16x2(tv[0], tv[1]);
      hi.y = pack_bf16x2(tv[2], tv[3]);
      hi.z = pack_bf16x2(tv[4], tv[5]);
      hi.w = pack_bf16x2(tv[6], tv[7]);
      lo.x = pack_bf16x2(tv[0] - bf16_lo(hi.x), tv[1] - bf16_hi(hi.x));
      lo.y = pack_bf16x2(tv[2] - bf16_lo(hi.y), tv[3] - bf16_hi(hi.y));
      lo.z = pack_bf16x2(tv[4] - bf16_lo(hi.z), tv[5] - bf16_hi(hi.z));
      lo.w = pack_bf16x2(tv[6] - bf16_lo(hi.w), tv[7] - bf16_hi(hi.w));
#pragma unroll
      for (int nt = 0; nt < kDecNT; ++nt) {
        f32x4 tmp = mfma16(as_bf16x8(hi), as_bf16x8(bop[nt][rs]), f32x4{0.f, 0.f, 0.f, 0.f});
        tmp = mfma16(as_bf16x8(lo), as_bf16x8(bop[nt][rs]), tmp);
        acc[nt] += bt.scale * tmp;
      }
    }
  }

  // lane (g, c) of tile nt holds y[4 g + v][nb0 + 16 nt + c]
  if (P.S == 1) {
    if (nb0 >= N) return;
#pragma unroll
    for (int nt = 0; nt < kDecNT; ++nt) {
      const int64_t n = nb0 + 16 * nt + c;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = 4 * g + v;
        if (m < M && n < N) P.y[m * N + n] = bf16_bits(acc[nt][v]);
      }
    }
    return;
  }
  // split K: partial sums [M][256] of this split, then the last split of the
  // row block to arrive adds all of them in split order. The partials and the
  // counter are written and read with device-scope atomic accesses, which are
  // coherent across the XCDs' L2 caches without writing back or invalidating
  // them (a device-scope fence would do both, for every workgroup); each wave
  // waits for its partial stores to complete before the workgroup barrier that
  // precedes the arrival increment.
  float* const part_rb = bt.part + (P.part0 + static_cast<int64_t>(b) * P.S) * (M * kDecRows);
  float* const mine = part_rb + static_cast<int64_t>(s) * (M * kDecRows);
#pragma unroll
  for (int nt = 0; nt < kDecNT; ++nt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * g + v;
      if (m < M)
        __hip_atomic_store(mine + m * kDecRows + 64 * w + 16 * nt + c, acc[nt][v], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);                  // this wave's stores have completed
  __syncthreads();
  if (t == 0) {
    const unsigned old = __hip_atomic_fetch_add(bt.cnt + P.cnt0 + b, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    last_flag = old == static_cast<unsigned>(P.S - 1);
  }
  __syncthreads();
  if (!last_flag) return;
  // thread t adds 4 consecutive outputs over the splits, eight splits' loads
  // in flight at a time; loads with the device-coherence bit (sc1) read what
  // other XCDs wrote
  const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
      part_rb, 0, static_cast<int>(P.S * M * kDecRows * 4), kDecBufWord3);
  const int64_t n0 = static_cast<int64_t>(b) * kDecRows;
  for (int i4 = t; i4 < M * kDecRows / 4; i4 += 256) {
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
    for (int sp0 = 0; sp0 < P.S; sp0 += 8) {
      f32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t off = static_cast<uint32_t>(((sp0 + u) * M * kDecRows + 4 * i4) * 4);
        v[u] = sp0 + u < P.S ? __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(prs, off, 0, 16))
                             : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) sum += v[u];
    }
    const int m = 4 * i4 / kDecRows, jn = 4 * i4 - m * kDecRows;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (n0 + jn + e < N) P.y[m * N + n0 + jn + e] = bf16_bits(sum[e]);
  }
  if (t == 0) __hip_atomic_store(bt.cnt + P.cnt0 + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
// The weights go in chunks of at most kDecMaxProblems, one launch each; the
// plan of a chunk depends only on that chunk.
DecChunkPlan dec_plan_chunk(int64_t M, int cn, const int64_t* N, const int64_t* K) {
  DecChunkPlan pl;
  int64_t rb_total = 0;
  for (int i = 0; i < cn; ++i) rb_total += cdiv(N[i], kDecRows);
  // about kDecTargetItems items per launch; a split covers at least two
  // super-steps (each split costs a round of fp32 partials and a fix-up)
  const int64_t s_all = rb_total >= kDecTargetItems / 2 ? 1 : cdiv(kDecTargetItems, rb_total);
  const int64_t min_sps = 2;
  for (int i = 0; i < cn; ++i) {
    const int64_t nss = cdiv(K[i] / 64, 4);
    int64_t S = s_all < nss ? s_all : nss;
    int64_t sps = cdiv(nss, S);
    if (sps < min_sps) sps = min_sps < nss ? min_sps : nss;
    if (sps > kDecMaxSps) sps = kDecMaxSps;     // bounded items balance the chip's load
    S = cdiv(nss, sps);
    const int64_t rb = cdiv(N[i], kDecRows);
    pl.S[i] = static_cast<int>(S);
    pl.sps[i] = static_cast<int>(sps);
    pl.items += rb * S;
    if (S > 1) {
      pl.slots += rb * S;
      pl.counters += rb;
    }
  }
  return pl;
}

size_t dec_workspace_bytes(int64_t M, int G, const int64_t* N, const int64_t* K) {
  int64_t max_slots = 0;
  for (int c0 = 0; c0 < G; c0 += kDecMaxProblems) {
    const int cn = G - c0 < kDecMaxProblems ? G - c0 : kDecMaxProblems;
    const DecChunkPlan pl = dec_plan_chunk(M, cn, N + c0, K + c0);
    if (pl.slots > max_slots) max_slots = pl.slots;
  }
  if (max_slots == 0) return 0;
  return kWsCounterBytes + align256(static_cast<size_t>(max_slots * M * kDecRows * 4));
}

hipError_t launch_dec_fwd(int64_t M, int G, const uint16_t* const* x, const int64_t* N, const int64_t* K,
                          const uint8_t* const* packed, const int8_t* const* qscale, const float* const* step,
                          const uint16_t* const* A, const uint16_t* const* B, int r, float alpha,
                          uint16_t* const* y, void* ws, const Codebook& cb, hipStream_t stream) {
  char* wsb = static_cast<char*>(ws);
  const int RT = r <= 0 ? 0 : r <= 16 ? 1 : r <= 32 ? 2 : r <= 64 ? 4 : 8;
  mark_kernel(0, stream);
  for (int c0 = 0; c0 < G; c0 += kDecMaxProblems) {
    const int cn = G - c0 < kDecMaxProblems ? G - c0 : kDecMaxProblems;
    const DecChunkPlan pl = dec_plan_chunk(M, cn, N + c0, K + c0);
    DecFwdBatch bt{};
    bt.count = cn;
    bt.M = static_cast<int>(M);
    bt.r = r;
    bt.scale = r > 0 ? alpha / static_cast<float>(r) : 0.0f;
    bt.cnt = pl.slots ? reinterpret_cast<unsigned*>(wsb) : nullptr;
    bt.part = pl.slots ? reinterpret_cast<float*>(wsb + kWsCounterBytes) : nullptr;
    int items = 0, slot = 0, cnt = 0;
    for (int i = 0; i < cn; ++i) {
      const int q = c0 + i;
      DecFwdProblem& P = bt.p[i];
      P.x = x[q];
      P.packed = packed[q];
      P.qscale = qscale[q];
      P.step = step[q];
      P.A = r > 0 ? A[q] : nullptr;
      P.B = r > 0 ? B[q] : nullptr;
      P.y = y[q];
      P.N = static_cast<int>(N[q]);
      P.K = static_cast<int>(K[q]);
      P.S = pl.S[i];
      P.sps = pl.sps[i];
      P.item0 = items;
      const int rb = static_cast<int>(cdiv(N[q], kDecRows));
      items += rb * P.S;
      P.part0 = slot;
      P.cnt0 = cnt;
      if (P.S > 1) {
        slot += rb * P.S;
        cnt += rb;
      }
    }
    bt.items = items;
    bool quad = true;
    for (int i = 0; i < cn; ++i) quad = quad && K[c0 + i] % 256 == 0;
    const dim3 grid(static_cast<unsigned>(round_up(items, 8)));
#define QNF4_DEC(RTV)                                                                    \
  if (quad)                                                                              \
    hipLaunchKernelGGL(HIP_KERNEL_NAME(k_dec_fwd<RTV, true>), grid, dim3(256), 0, stream, bt, cb); \
  else                                                                                   \
    hipLaunchKernelGGL(HIP_KERNEL_NAME(k_dec_fwd<RTV, false>), grid, dim3(256), 0, stream, bt, cb)
    switch (RT) {
      case 0: QNF4_DEC(0); break;
      case 1: QNF4_DEC(1); break;
      case 2: QNF4_DEC(2); break;
      case 4: QNF4_DEC(4); break;
      default: QNF4_DEC(8); break;
    }
#undef QNF4_DEC
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  mark_kernel(1, stream);
  return hipSuccess;
}

}  // namespace qnf4
