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
// (a contraction does not depend on the order of its terms). About 19 VALU
// operations per 8 weights.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "mm_common.hpp"

namespace qnf4 {

// entry j (0..7) = bf16(L[15 - j] * s): the magnitudes, largest first; low and
// high bytes in separate planes of two dwords each
struct PermTable {
  uint32_t lo0, lo1, hi0, hi1;
};

__device__ __forceinline__ PermTable make_ptable(const Codebook& cb, float s) {
  const uint32_t p0 = pack_bf16x2(cb.L[15] * s, cb.L[14] * s);
  const uint32_t p1 = pack_bf16x2(cb.L[13] * s, cb.L[12] * s);
  const uint32_t p2 = pack_bf16x2(cb.L[11] * s, cb.L[10] * s);
  const uint32_t p3 = pack_bf16x2(cb.L[9] * s, cb.L[8] * s);
  PermTable t;
  t.lo0 = perm(p1, p0, 0x06040200u);
  t.hi0 = perm(p1, p0, 0x07050301u);
  t.lo1 = perm(p3, p2, 0x06040200u);
  t.hi1 = perm(p3, p2, 0x07050301u);
  return t;
}

// One packed word (8 codes, element 2i in the low nibble of byte i) -> 8 bf16
// in the order 0 2 | 4 6 | 1 3 | 5 7 (pairs per dword, low half first).
__device__ __forceinline__ u32x4 decode8_perm(uint32_t d, const PermTable& t) {
  const uint32_t n8 = d & 0x88888888u;                   // bit 3 of every code
  const uint32_t x = d ^ (n8 - (n8 >> 3));               // c XOR 7b per nibble
  const uint32_t se = x & 0x07070707u;                   // magnitude index, even elements
  const uint32_t so = (x >> 4) & 0x07070707u;            // odd elements
  const uint32_t nd = ~d;                                // bit 3 clear <=> negative level
  const uint32_t loE = perm(t.lo1, t.lo0, se);
  const uint32_t hiE = perm(t.hi1, t.hi0, se) | ((nd << 4) & 0x80808080u);
  const uint32_t loO = perm(t.lo1, t.lo0, so);
  const uint32_t hiO = perm(t.hi1, t.hi0, so) | (nd & 0x80808080u);
  u32x4 r;
  r.x = perm(hiE, loE, 0x05010400u);
  r.y = perm(hiE, loE, 0x07030602u);
  r.z = perm(hiO, loO, 0x05010400u);
  r.w = perm(hiO, loO, 0x07030602u);
  return r;
}

// 8 consecutive bf16 (4 dwords, low half first) -> the order 0 2 | 4 6 | 1 3 | 5 7
__device__ __forceinline__ u32x4 perm8(const u32x4& v) {
  u32x4 r;
  r.x = perm(v.y, v.x, 0x05040100u);
  r.y = perm(v.w, v.z, 0x05040100u);
  r.z = perm(v.y, v.x, 0x07060302u);
  r.w = perm(v.w, v.z, 0x07060302u);
  return r;
}

constexpr int kDecNT = 4;                         // 16-row MFMA tiles per wave
constexpr int kDecBufWord3 = 0x00020000;          // raw buffer descriptor word 3 on gfx9-family parts
constexpr int kDecRows = 16 * kDecNT * 4;         // weight rows per item (four waves)

__device__ __forceinline__ int dec_item_of(int wg, int grid) {
  // grid is a multiple of 8: XCD (wg % 8) gets items [xcd * grid/8, ...)
  return (wg & 7) * (grid >> 3) + (wg >> 3);
}

// RT: rank tiles of 16 the kernel computes (0: no adapter; else a power of two
// with 16 RT >= r). For r <= 16 the adapter rows travel with the stage.
template <int RT>
struct DecStage {
  static constexpr int kPF = 1;
  u32x4 cw[kDecNT][2];   // codes: the lane's block of each tile's weight row
  u32x4 xa[8];           // 64 activations of x row c (natural order, then permuted)
  u32x4 af[kPF][2];      // adapter rows for this wave's two MFMAs of t
  float d[kDecNT];
  int8_t q[kDecNT];
};

template <int RT>
__global__ __launch_bounds__(256, 2) void k_dec_fwd(DecFwdBatch bt, Codebook cb) {
  constexpr int kRT = RT > 0 ? RT : 1;
  constexpr int kRS = RT > 1 ? RT / 2 : 1;      // 32-deep rank chunks of the up-projection
  constexpr bool kPrefetchA = RT == 1;
  __shared__ float tsh[RT > 0 ? 4 * 16 * (16 * kRT + 4) : 1];
  __shared__ int last_flag;

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
  const int64_t N = P.N, K = P.K;
  const int64_t nbr = K / 64, nss = cdiv(nbr, 4);
  const int local = item - P.item0;
  const int b = local / P.S, s = local - (local / P.S) * P.S;
  const int64_t ss0 = static_cast<int64_t>(s) * P.sps;
  const int64_t ss1 = imin(ss0 + P.sps, nss);
  const int64_t nb0 = static_cast<int64_t>(b) * kDecRows + 64 * w;   // this wave's first row

  // every load is unconditional (rows past N re-read row N - 1 and are never
  // stored; x rows past M and adapter rows past r read as zero through the
  // buffer descriptors' range checks), so the only branches of the loop are
  // uniform loop control and the compiler can keep the next stage in flight
  const uint8_t* prow[kDecNT];
  int64_t bix[kDecNT];
#pragma unroll
  for (int nt = 0; nt < kDecNT; ++nt) {
    const int64_t n = imin(nb0 + 16 * nt + c, N - 1);
    prow[nt] = P.packed + n * (K / 2);
    bix[nt] = n * nbr;
  }
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(P.x), 0, static_cast<int>(M * K * 2), kDecBufWord3);
  const uint32_t xoff = static_cast<uint32_t>(c * K * 2);
  const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(RT > 0 ? P.A : P.x), 0, static_cast<int>(RT > 0 ? r * K * 2 : 0), kDecBufWord3);

  // adapter rows 16 jt + c of block 4 ss + g, 8-element pieces 2w and 2w + 1
  // (wave w computes those two MFMAs of t; past K they read as zero)
  auto load_adapter = [&](int64_t ss, int jt, u32x4 (&af)[2]) {
    const int64_t kbr = ss * 4 + g;
    const int64_t kb = imin(kbr, nbr - 1);
    const uint32_t off = kbr < nbr ? static_cast<uint32_t>(((16 * jt + c) * K + kb * 64 + 16 * w) * 2) : 0x80000000u;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      af[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ars, off + 16 * i, 0, 0));
  };
  // activations first: the end of the previous super-step waits for them
  // (and permutes them in place) while the codes stay in flight
  auto load = [&](int64_t ss, DecStage<RT>& st) {
    const int64_t kb = imin(ss * 4 + g, nbr - 1);
    const uint32_t xo = xoff + static_cast<uint32_t>(kb * 128);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      st.xa[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, xo + 16 * j, 0, 0));
#pragma unroll
    for (int nt = 0; nt < kDecNT; ++nt) {
      st.cw[nt][0] = ld16(prow[nt] + kb * 32);
      st.cw[nt][1] = ld16(prow[nt] + kb * 32 + 16);
      st.q[nt] = P.qscale[bix[nt] + kb];
      st.d[nt] = P.step[(bix[nt] + kb) >> 8];
    }
    if constexpr (kPrefetchA) {
#pragma unroll
      for (int jt = 0; jt < RT; ++jt) load_adapter(ss, jt, st.af[jt]);
    }
  };
  auto permute_x = [&](DecStage<RT>& st) {
#pragma unroll
    for (int j = 0; j < 8; ++j) st.xa[j] = perm8(st.xa[j]);
  };

  f32x4 acc[kDecNT], tacc[kRT];
#pragma unroll
  for (int nt = 0; nt < kDecNT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int jt = 0; jt < kRT; ++jt) tacc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one super-step on `cur`; with kPre the next one is requested into `nxt`
  // first (and its activations permuted at the end). Larger ranks request
  // their adapter rows before the next stage, so that waiting for them leaves
  // the stage in flight.
  auto body = [&](auto pre, int64_t ss, const DecStage<RT>& cur, DecStage<RT>& nxt) {
    constexpr bool kPre = decltype(pre)::value;
    const bool kvalid = ss * 4 + g < nbr;
    u32x4 afl[2];
    if constexpr (RT > 0 && !kPrefetchA) load_adapter(ss, 0, afl);
    if constexpr (kPre) load(ss + 1, nxt);
#pragma unroll
    for (int nt = 0; nt < kDecNT; ++nt) {
      const float sc = kvalid ? block_scale(cur.q[nt], cur.d[nt]) : 0.0f;
      const PermTable tb = make_ptable(cb, sc);
      const uint32_t pw[8] = {cur.cw[nt][0].x, cur.cw[nt][0].y, cur.cw[nt][0].z, cur.cw[nt][0].w,
                              cur.cw[nt][1].x, cur.cw[nt][1].y, cur.cw[nt][1].z, cur.cw[nt][1].w};
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[nt] = mfma16(as_bf16x8(cur.xa[j]), as_bf16x8(decode8_perm(pw[j], tb)), acc[nt]);
    }
    if constexpr (RT > 0) {
      // pieces 2w, 2w + 1 of the lane's 64 activations (wave-uniform index)
      const u32x4 x0 = w == 0 ? cur.xa[0] : w == 1 ? cur.xa[2] : w == 2 ? cur.xa[4] : cur.xa[6];
      const u32x4 x1 = w == 0 ? cur.xa[1] : w == 1 ? cur.xa[3] : w == 2 ? cur.xa[5] : cur.xa[7];
      if constexpr (kPrefetchA) {
#pragma unroll
        for (int jt = 0; jt < RT; ++jt) {
          tacc[jt] = mfma16(as_bf16x8(x0), as_bf16x8(perm8(cur.af[jt][0])), tacc[jt]);
          tacc[jt] = mfma16(as_bf16x8(x1), as_bf16x8(perm8(cur.af[jt][1])), tacc[jt]);
        }
      } else {
#pragma unroll
        for (int jt = 0; jt < kRT; ++jt) {
          if (jt > 0) load_adapter(ss, jt, afl);
          tacc[jt] = mfma16(as_bf16x8(x0), as_bf16x8(perm8(afl[0])), tacc[jt]);
          tacc[jt] = mfma16(as_bf16x8(x1), as_bf16x8(perm8(afl[1])), tacc[jt]);
        }
      }
    }
    if constexpr (kPre) permute_x(nxt);
  };

  using Pre = std::integral_constant<bool, true>;
  using NoPre = std::integral_constant<bool, false>;
  DecStage<RT> st0, st1;
  if (ss0 < ss1) {
    load(ss0, st0);
    permute_x(st0);
  }
  int64_t ss = ss0;
  for (; ss + 2 < ss1; ss += 2) {
    body(Pre{}, ss, st0, st1);
    body(Pre{}, ss + 1, st1, st0);
  }
  if (ss + 1 < ss1) {
    body(Pre{}, ss, st0, st1);
    body(NoPre{}, ss + 1, st1, st0);
  } else if (ss < ss1) {
    body(NoPre{}, ss, st0, st1);
  }

  // LoRA: sum the four waves' parts of t (fixed order), then add
  // scale * (t_hi + t_lo) . B^T to each tile
  if (RT > 0) {
    constexpr int kLd = 16 * kRT + 4;
    u32x4 bop[kDecNT][kRS];
#pragma unroll
    for (int nt = 0; nt < kDecNT; ++nt) {
      const int64_t n = imin(nb0 + 16 * nt + c, N - 1);
#pragma unroll
      for (int rs = 0; rs < kRS; ++rs)
        bop[nt][rs] = load_row8(P.B + n * r, 32 * rs + 8 * g, r, (r & 7) == 0);
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
  const int64_t n0 = static_cast<int64_t>(b) * kDecRows;
  for (int idx = t; idx < M * kDecRows; idx += 256) {
    const int m = idx / kDecRows, jn = idx - m * kDecRows;
    float sum = 0.f;
    for (int sp = 0; sp < P.S; ++sp)
      sum += __hip_atomic_load(part_rb + sp * (M * kDecRows) + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (n0 + jn < N) P.y[m * N + n0 + jn] = bf16_bits(sum);
  }
  if (t == 0) __hip_atomic_store(bt.cnt + P.cnt0 + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
DecPlan dec_plan(int64_t M, int G, const int64_t* N, const int64_t* K) {
  DecPlan pl;
  pl.S.assign(G, 1);
  pl.sps.assign(G, 1);
  // chunks of at most kDecMaxProblems weights, one launch each; the plan of a
  // chunk depends only on that chunk
  for (int c0 = 0; c0 < G; c0 += kDecMaxProblems) {
    const int cn = G - c0 < kDecMaxProblems ? G - c0 : kDecMaxProblems;
    int64_t rb_total = 0;
    for (int i = 0; i < cn; ++i) rb_total += cdiv(N[c0 + i], kDecRows);
    // about kDecTargetItems items per launch; at M > 4 a split covers at least
    // two super-steps (its fp32 partials are M KB per 256 rows)
    const int64_t s_all = rb_total >= kDecTargetItems / 2 ? 1 : cdiv(kDecTargetItems, rb_total);
    const int64_t min_sps = M > 4 ? 2 : 1;
    int64_t items = 0, slots = 0, counters = 0;
    for (int i = 0; i < cn; ++i) {
      const int64_t nss = cdiv(K[c0 + i] / 64, 4);
      int64_t S = s_all < nss ? s_all : nss;
      int64_t sps = cdiv(nss, S);
      if (sps < min_sps) sps = min_sps < nss ? min_sps : nss;
      S = cdiv(nss, sps);
      const int64_t rb = cdiv(N[c0 + i], kDecRows);
      pl.S[c0 + i] = static_cast<int>(S);
      pl.sps[c0 + i] = static_cast<int>(sps);
      items += rb * S;
      if (S > 1) {
        slots += rb * S;
        counters += rb;
      }
    }
    if (slots > pl.max_slots) pl.max_slots = slots;
    if (counters > pl.max_counters) pl.max_counters = counters;
    if (items > pl.max_items) pl.max_items = items;
  }
  pl.part_bytes = align256(static_cast<size_t>(pl.max_slots * M * kDecRows * 4));
  return pl;
}

size_t dec_workspace_bytes(int64_t M, int G, const int64_t* N, const int64_t* K) {
  const DecPlan pl = dec_plan(M, G, N, K);
  if (pl.max_slots == 0) return 0;
  return kWsCounterBytes + pl.part_bytes;
}

hipError_t launch_dec_fwd(int64_t M, int G, const uint16_t* const* x, const int64_t* N, const int64_t* K,
                          const uint8_t* const* packed, const int8_t* const* qscale, const float* const* step,
                          const uint16_t* const* A, const uint16_t* const* B, int r, float alpha,
                          uint16_t* const* y, void* ws, const Codebook& cb, hipStream_t stream) {
  const DecPlan pl = dec_plan(M, G, N, K);
  char* wsb = static_cast<char*>(ws);
  const int RT = r <= 0 ? 0 : r <= 16 ? 1 : r <= 32 ? 2 : r <= 64 ? 4 : 8;
  for (int c0 = 0; c0 < G; c0 += kDecMaxProblems) {
    const int cn = G - c0 < kDecMaxProblems ? G - c0 : kDecMaxProblems;
    DecFwdBatch bt{};
    bt.count = cn;
    bt.M = static_cast<int>(M);
    bt.r = r;
    bt.scale = r > 0 ? alpha / static_cast<float>(r) : 0.0f;
    bt.cnt = pl.max_slots ? reinterpret_cast<unsigned*>(wsb) : nullptr;
    bt.part = pl.max_slots ? reinterpret_cast<float*>(wsb + kWsCounterBytes) : nullptr;
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
      P.S = pl.S[q];
      P.sps = pl.sps[q];
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
    const dim3 grid(static_cast<unsigned>(round_up(items, 8)));
#define QNF4_DEC(RTV) hipLaunchKernelGGL(k_dec_fwd<RTV>, grid, dim3(256), 0, stream, bt, cb)
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
  return hipSuccess;
}

}  // namespace qnf4
