// Adapter gradients of one QLoRA linear for gfx950. Only the adapters train:
// the base is frozen and gradients and optimizer state exist for A and B alone
// ("QLoRA Explained", "What is QLoRA?"; "QLoRA and Quantized Training", "The
// idea"; "A 65B fine-tune on the GPU you already have", figure 2). With
// s = alpha / r, t = bf16(x . A^T) and u = bf16(dY . B) (the same bf16 values
// the fused forward and backward use):
//     dB [N, r] = s . dY^T . t        dA [r, K] = s . u^T . x
// Both are a contraction over the M tokens of a wide bf16 matrix P [M, C]
// (dY or x) with a rank-r one Q [M, r] (t or u): G = P^T . Q. P is read once
// from HBM and Q stays in L2, so the kernel is HBM-bound (r MACs per element
// of P); the products run on 16x16x32 bf16 MFMA with fp32 accumulation.
//
// k_lora_grad: workgroup = 64 columns of P x one of S row splits; wave w owns
//   16 columns. Rows go in chunks of 64: each thread loads two 16-byte pieces
//   of the chunk into registers two chunks ahead, writes them into a
//   double-buffered LDS tile (bank-swizzled) and the waves read their MFMA
//   operands P[m .. m+7][c] transposed with ds_read_b64_tr_b16. Q is stored
//   transposed (Qt [rp][Mp], zero past M), so its operands are plain 16-byte
//   loads from L2. Each split writes fp32 partials.
// k_grad_finish: sums the S partials in order (deterministic), scales by s and
//   writes or accumulates into dA / dB.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "mm_common.hpp"

namespace qnf4 {

namespace {

constexpr int kGradCols = 64;      // columns of P per workgroup
constexpr int kGradRows = 64;      // rows of P per chunk
constexpr int kGradWGs = 512;      // target workgroups per contraction

// s_waitcnt vmcnt(n) / lgkmcnt(0) (gfx9 encoding), and a barrier without the
// vmcnt(0) that __syncthreads' fence implies (register prefetches stay in
// flight across it)
constexpr int grad_vmcnt(int n) { return ((n >> 4) << 14) | 0x0F70 | (n & 15); }
template <int N>
__device__ __forceinline__ void grad_wait_vm() { __builtin_amdgcn_s_waitcnt(grad_vmcnt(N)); }
__device__ __forceinline__ void grad_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("s_barrier" ::: "memory");
}

// LDS tile: 64 rows x 8 chunks of 16 bytes. Chunk c of row m sits at
// c ^ 2 f(m), f(m) = ((m >> 3) & 3) ^ ((m >> 1) & 1): a transposed read of 4
// rows at row offsets 8G + 4q + (0..3), G = 0..3, then touches each bank
// exactly twice.
__device__ __forceinline__ int grad_swz(int m) { return 2 * (((m >> 3) & 3) ^ ((m >> 1) & 1)); }

}  // namespace

// P [M][C] bf16 (C % 8 == 0, rows 16-byte aligned); Qt [16 NT][Mp] bf16 (Mp
// a multiple of 64, rows past M zero; ranks past r arbitrary). P and Qt are deliberately not
// __restrict__: with it the compiler may sink the prefetch loads past the
// barriers to their use (the asm barrier is then not known to order them). Split s covers chunks [s n / S, (s+1) n / S)
// of n = Mp / 64. TR == false: part[s][c][r] (the dB layout); TR == true:
// part[s][j][C] (the dA layout).
template <int NT, bool TR>
__global__ __launch_bounds__(256) void k_lora_grad(const uint16_t* P, int64_t M, int64_t C,
                                                   const uint16_t* Qt, int64_t Mp, int r,
                                                   int ctiles, int S, float* __restrict__ part) {
  __shared__ u32x4 tile[2][kGradRows * 8];
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int ct = blockIdx.x % ctiles, s = blockIdx.x / ctiles;
  const int64_t c0 = static_cast<int64_t>(ct) * kGradCols;
  const int64_t nch = Mp / kGradRows;
  const int64_t ch0 = s * nch / S, ch1 = (s + 1) * nch / S;

  // this thread's two 16-byte pieces of a chunk: rows lr and lr + 32, chunk
  // lc, through a buffer descriptor over the split's rows starting at column
  // c0: rows past M read as zero; a piece past column C reads the next row
  // (finite data, and only into output columns >= C, which are not stored)
  const int lr = t >> 3, lc = t & 7;
  const int64_t row0 = ch0 * kGradRows;
  const int64_t rows_valid = imin(M, ch1 * kGradRows) - row0;
  const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(P + row0 * C + c0), 0, static_cast<int>((rows_valid * C - c0) * 2), 0x00020000);
  uint32_t poff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) poff[i] = static_cast<uint32_t>(((lr + 32 * i) * C + 8 * lc) * 2);
  // operand lanes: G = lane / 16 takes rows 8G .. 8G + 7 of a 32-row k-step,
  // j16 = lane % 16 is the column (of P) or the rank (of Q) it serves
  const int G = lane >> 4, j16 = lane & 15;

  struct Regs {
    u32x4 p[2];
    u32x4 q[2][NT];
  };
  auto load = [&](int64_t ch, Regs& R) {
    const int64_t mb = ch * kGradRows;
    const uint32_t so = static_cast<uint32_t>((mb - row0) * C * 2);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      R.p[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(pr, poff[i], so, 0));
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int jt = 0; jt < NT; ++jt)
        R.q[kk][jt] = ld16(Qt + (16 * jt + j16) * Mp + mb + 32 * kk + 8 * G);
  };
  auto store = [&](const Regs& R, u32x4* T) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int m = lr + 32 * i;
      T[m * 8 + (lc ^ grad_swz(m))] = R.p[i];
    }
  };
  f32x4 acc[NT];
#pragma unroll
  for (int jt = 0; jt < NT; ++jt) acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the P operand of k-step kk: rows 32 kk + 8G + 4q + (j16 >> 2), 4 columns
  // at 4 (j16 & 3) of the wave's 16
  auto compute = [&](const Regs& R, const u32x4* T) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      s16x4 v[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int m = 32 * kk + 8 * G + 4 * q + (j16 >> 2);
        const int col = 16 * w + 4 * (j16 & 3);             // bf16 column within the 64
        const int chunk = (col >> 3) ^ grad_swz(m);
        v[q] = ds_read_tr(T, (m * 8 + chunk) * 8 + (col & 7));
      }
      const bf16x8 pa = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int jt = 0; jt < NT; ++jt) {
        const bf16x8 qb = as_bf16x8(R.q[kk][jt]);
        acc[jt] = TR ? mfma16(qb, pa, acc[jt]) : mfma16(pa, qb, acc[jt]);
      }
    }
  };

  // three register sets, chunk ch in set (ch - ch0) % 3; loads past the
  // split's end re-read its last chunk so that every iteration has the same
  // number of loads in flight
  constexpr int kLoads = 2 + 2 * NT;        // vector loads per chunk per thread
  Regs R0, R1, R2;
  const int64_t last = ch1 - 1;
  load(ch0, R0);
  load(ch0 + 1 <= last ? ch0 + 1 : last, R1);
  int64_t ch = ch0;
  auto step = [&](Regs& cur, Regs& nxt2, int buf) {
    load(ch + 2 <= last ? ch + 2 : last, nxt2);
    grad_wait_vm<2 * kLoads>();             // chunk ch has landed
    store(cur, tile[buf]);
    grad_barrier();                         // (also: every wave is done with tile[buf] of chunk ch - 2)
    compute(cur, tile[buf]);
    ++ch;
  };
  while (ch < ch1) {
    step(R0, R2, 0);
    if (ch >= ch1) break;
    step(R1, R0, 1);
    if (ch >= ch1) break;
    step(R2, R1, 0);
    if (ch >= ch1) break;
    step(R0, R2, 1);
    if (ch >= ch1) break;
    step(R1, R0, 0);
    if (ch >= ch1) break;
    step(R2, R1, 1);
  }

  // partials: mfma16 output lane holds rows 4G + v, column j16 of the 16 x 16
  // tile (rows = P columns for TR == false, ranks for TR == true)
  float* out = part + static_cast<int64_t>(s) * C * r;
#pragma unroll
  for (int jt = 0; jt < NT; ++jt)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      if (TR) {
        const int j = 16 * jt + 4 * G + v;
        const int64_t c = c0 + 16 * w + j16;
        if (j < r && c < C) out[j * C + c] = acc[jt][v];
      } else {
        const int64_t c = c0 + 16 * w + 4 * G + v;
        const int j = 16 * jt + j16;
        if (j < r && c < C) out[c * r + j] = acc[jt][v];
      }
    }
}

// out[i] = (accumulate ? out[i] : 0) + scale * sum_s part[s][i], for two arrays
// (dB then dA) in one launch; n0 and n1 are multiples of 4.
__global__ __launch_bounds__(256) void k_grad_finish(const float* __restrict__ p0, int S0, int64_t n0,
                                                     float* __restrict__ o0, const float* __restrict__ p1, int S1,
                                                     int64_t n1, float* __restrict__ o1, float scale,
                                                     int accumulate) {
  int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  const float* p = p0;
  float* o = o0;
  int S = S0;
  int64_t n = n0;
  if (i >= n0) {
    i -= n0;
    p = p1, o = o1, S = S1, n = n1;
    if (i >= n1) return;
  }
  f32x4 sum = *reinterpret_cast<const f32x4*>(p + i);
  for (int s = 1; s < S; ++s) sum += *reinterpret_cast<const f32x4*>(p + s * n + i);
  sum *= scale;
  f32x4* dst = reinterpret_cast<f32x4*>(o + i);
  if (accumulate) sum += *dst;
  *dst = sum;
}

GradPlan grad_plan(int64_t M, int64_t N, int64_t K, int r) {
  GradPlan g;
  g.Mp = round_up(M, kGradRows);
  g.rp = rank_pad(r);
  const int64_t nch = g.Mp / kGradRows;
  // enough splits for about kGradWGs workgroups, and for each split's rows of
  // P to span less than 1 GiB (32-bit buffer offsets); at most one per chunk
  auto splits = [&](int64_t C) {
    const int64_t ct = cdiv(C, kGradCols);
    int64_t s = cdiv(kGradWGs, ct);
    const int64_t smin = cdiv(g.Mp * C * 2, int64_t{1} << 30);
    if (s < smin) s = smin;
    if (s > nch) s = nch;
    return s < 1 ? int64_t{1} : s;
  };
  g.SB = splits(N);
  g.SA = splits(K);
  size_t off = kWsCounterBytes;                 // the workspace's counter region is left alone
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  g.bt_off = take(static_cast<size_t>(r) * N * 2);
  // rows of t^T / u^T: the rank tiles the gradient kernel reads (16 NT, NT the
  // power of two >= ceil(r / 16)) may exceed rp; rows past rp are never
  // written and feed only output ranks >= r, which are not stored
  const int64_t rows = std::max<int64_t>(g.rp, 16 * down_nt(r));
  g.tt_off = take(static_cast<size_t>(rows) * g.Mp * 2);
  g.ut_off = take(static_cast<size_t>(rows) * g.Mp * 2);
  g.pb_off = take(static_cast<size_t>(g.SB) * N * r * 4);
  g.pa_off = take(static_cast<size_t>(g.SA) * K * r * 4);
  g.dp_off = take(std::max(down_plan(M, K, r).part_bytes, down_plan(M, N, r).part_bytes));
  g.total = off;
  return g;
}

hipError_t launch_lora_grad(const uint16_t* x, const uint16_t* dy, int64_t M, int64_t N, int64_t K,
                            const uint16_t* A, const uint16_t* B, int r, float alpha, float* dA, float* dB,
                            int accumulate, void* ws, hipStream_t stream) {
  const GradPlan g = grad_plan(M, N, K, r);
  char* wsb = static_cast<char*>(ws);
  uint16_t* bt = reinterpret_cast<uint16_t*>(wsb + g.bt_off);
  uint16_t* tt = reinterpret_cast<uint16_t*>(wsb + g.tt_off);
  uint16_t* ut = reinterpret_cast<uint16_t*>(wsb + g.ut_off);
  float* pb = reinterpret_cast<float*>(wsb + g.pb_off);
  float* pa = reinterpret_cast<float*>(wsb + g.pa_off);
  float* dp = reinterpret_cast<float*>(wsb + g.dp_off);
  hipError_t e = launch_lora_down(true, x, M, K, A, r, tt, stream, nullptr, dp, g.Mp);     // t^T [rp][Mp]
  if (e != hipSuccess) return e;
  e = launch_lora_down(false, dy, M, N, B, r, ut, stream, bt, dp, g.Mp);                  // u^T [rp][Mp]
  if (e != hipSuccess) return e;
  const int ctb = static_cast<int>(cdiv(N, kGradCols)), cta = static_cast<int>(cdiv(K, kGradCols));
  const int SB = static_cast<int>(g.SB), SA = static_cast<int>(g.SA);
  const int nt = down_nt(r);
#define QNF4_GRAD(NTV)                                                                                         \
  do {                                                                                                         \
    hipLaunchKernelGGL(HIP_KERNEL_NAME(k_lora_grad<NTV, false>), dim3(ctb * SB), dim3(256), 0, stream, dy, M, N, \
                       tt, g.Mp, r, ctb, SB, pb);                                                              \
    hipLaunchKernelGGL(HIP_KERNEL_NAME(k_lora_grad<NTV, true>), dim3(cta * SA), dim3(256), 0, stream, x, M, K,   \
                       ut, g.Mp, r, cta, SA, pa);                                                              \
  } while (0)
  if (nt <= 1)
    QNF4_GRAD(1);
  else if (nt == 2)
    QNF4_GRAD(2);
  else if (nt <= 4)
    QNF4_GRAD(4);
  else
    QNF4_GRAD(8);
#undef QNF4_GRAD
  const int64_t nb = N * r, na = static_cast<int64_t>(r) * K;
  const unsigned grid = static_cast<unsigned>(cdiv((nb + na) / 4, 256));
  hipLaunchKernelGGL(k_grad_finish, dim3(grid), dim3(256), 0, stream, pb, SB, nb, dB, pa, SA, na, dA,
                     alpha / static_cast<float>(r), accumulate);
  return hipGetLastError();
}

}  // namespace qnf4
