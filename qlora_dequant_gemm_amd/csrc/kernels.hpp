// Host-side launchers of the gfx950 kernels and the launch plan they share
// with the workspace query. Sizes are validated by the C ABI layer before any
// of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "codebook.hpp"

namespace qnf4 {

// M at or below this uses the GEMV-shaped kernels (decode shapes).
constexpr int64_t kSmallM = 16;

// Every workspace that is used at all starts with this many bytes of arrival
// counters (split-K fix-ups): zero before a call, left zero by every call.
// The other parts of a workspace layout follow it.
constexpr size_t kWsCounterBytes = 16384;

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ inline int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }
inline size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

// LoRA rank padded to the 32-deep MFMA contraction used by the epilogues.
inline int64_t rank_pad(int r) { return round_up(r, 32); }

// ---------------------------------------------------------------------------
// Decode-shaped forward (M <= kSmallM) over a table of weights: one launch per
// chunk of kDecMaxProblems weights (the table travels in the kernel
// arguments). Items are 256 weight rows x S_p ranges of K.
// ---------------------------------------------------------------------------
constexpr int kDecMaxProblems = 32;
constexpr int kMaxGroups = 8;             // weights of one grouped (shared-x) forward
constexpr int64_t kDecTargetItems = 1024;

// Tiled forward (M > kSmallM) over a table of weights in one launch; tile
// columns of weight i are [col0[i], col0[i + 1]) of the launch's sequence.
constexpr int kFwdMaxWeights = 8;
struct FwdTable {
  const uint16_t* x[kFwdMaxWeights];        // [M][K[i]]
  const uint8_t* packed[kFwdMaxWeights];
  const int8_t* qscale[kFwdMaxWeights];
  const float* step[kFwdMaxWeights];
  const uint16_t* tl[kFwdMaxWeights];       // t = bf16(x . A^T) [M][rp], or null
  const uint16_t* B[kFwdMaxWeights];        // [N[i]][r], or null
  uint16_t* y[kFwdMaxWeights];              // [M][N[i]]
  int N[kFwdMaxWeights], K[kFwdMaxWeights];
  int col0[kFwdMaxWeights + 1];
  int count;
};

struct DecFwdProblem {
  const uint16_t* x;        // [M][K]
  const uint8_t* packed;    // stored weight [N][K]
  const int8_t* qscale;
  const float* step;
  const uint16_t* A;        // [r][K] (r > 0)
  const uint16_t* B;        // [N][r]
  uint16_t* y;              // [M][N]
  int N, K;
  int item0, S, sps;        // first item; K splits; 256-deep super-steps per split
  int part0, cnt0;          // first partial slot and counter (S > 1)
};
struct DecFwdBatch {
  DecFwdProblem p[kDecMaxProblems];
  int count, items, M, r;
  float scale;
  float* part;              // [slots][M][256] fp32 partial sums
  unsigned* cnt;            // arrival counters, one per split row block
};
// Plan of one launch (at most kDecMaxProblems weights): splits of K per
// weight, super-steps per split, and the workspace slots and counters used.
struct DecChunkPlan {
  int S[kDecMaxProblems], sps[kDecMaxProblems];
  int64_t slots = 0, counters = 0, items = 0;
  bool wide = false;        // decode-shaped backward: the item shape
};
DecChunkPlan dec_plan_chunk(int64_t M, int cn, const int64_t* N, const int64_t* K);
size_t dec_workspace_bytes(int64_t M, int G, const int64_t* N, const int64_t* K);
// x[i], y[i] etc. are the G weights' operands (host arrays of device pointers)
hipError_t launch_dec_fwd(int64_t M, int G, const uint16_t* const* x, const int64_t* N, const int64_t* K,
                          const uint8_t* const* packed, const int8_t* const* qscale, const float* const* step,
                          const uint16_t* const* A, const uint16_t* const* B, int r, float alpha,
                          uint16_t* const* y, void* ws, const Codebook& cb, hipStream_t stream);

// Decode-shaped backward (M <= kSmallM) over a table of weights, one launch
// per chunk of kDecMaxProblems. A launch whose weights have fewer than
// kDbWideMin 256-column ranges in all runs narrow items (64 columns x S_p
// ranges of the weight's rows, at least kDbMinSps 64-row sub-tiles each,
// about kDbTargetItems items); larger launches run wide items (256 columns x
// at most kDwMaxSps super-steps of 256 rows, about kDbWideTarget items).
constexpr int64_t kDbWideMin = 128;
constexpr int64_t kDbMinSps = 8;
constexpr int64_t kDbTargetItems = 1024;
constexpr int kDwMaxSps = 4;
constexpr int64_t kDbWideTarget = 512;
struct DecBwdProblem {
  const uint16_t* dy;       // [M][N]
  const uint8_t* packed;    // stored weight [N][K]
  const int8_t* qscale;
  const float* step;
  const uint16_t* A;        // [r][K] (r > 0)
  const uint16_t* B;        // [N][r]
  uint16_t* dx;             // [M][K]
  int N, K;
  int item0, S, sps;        // first item; row splits; sub-tiles (narrow) or super-steps (wide) per split
  int part0, cnt0;          // first partial slot and counter (S > 1)
};
struct DecBwdBatch {
  DecBwdProblem p[kDecMaxProblems];
  int count, items, M, r;
  float scale;
  float* part;              // [slots][64 or 256 columns][M rounded up to 4] fp32 partial sums
  unsigned* cnt;            // arrival counters, one per split column range
};
DecChunkPlan dec_bwd_plan_chunk(int64_t M, int cn, const int64_t* N, const int64_t* K);
size_t dec_bwd_workspace_bytes(int64_t M, int G, const int64_t* N, const int64_t* K);
hipError_t launch_dec_bwd(int64_t M, int G, const uint16_t* const* dy, const int64_t* N, const int64_t* K,
                          const uint8_t* const* packed, const int8_t* const* qscale, const float* const* step,
                          const uint16_t* const* A, const uint16_t* const* B, int r, float alpha,
                          uint16_t* const* dx, void* ws, const Codebook& cb, hipStream_t stream);

// Tiled down-projection (M > kSmallM, and the adapter gradients): 64-row tiles
// x KS splits of the contraction, `sps` 32-deep steps each; with KS > 1 the
// splits write fp32 partials [KS][Mr][16 nt] (Mr = M rounded up to 64) that a
// second kernel sums in order. nt = rank tiles of 16 the kernel computes (a
// power of two >= ceil(r / 16)).
struct DownPlan {
  int64_t KS = 1, sps = 0, Mr = 0;
  int nt = 1;
  size_t part_bytes = 0;
};
inline int down_nt(int r) {
  const int n = (r + 15) / 16;
  return n <= 1 ? 1 : n == 2 ? 2 : n <= 4 ? 4 : 8;
}
inline DownPlan down_plan(int64_t M, int64_t Kc, int r) {
  DownPlan p;
  p.nt = down_nt(r);
  const int64_t tiles = cdiv(M, 64), nsteps = cdiv(Kc, 32);
  int64_t ks = cdiv(256, tiles);               // about one workgroup per CU
  const int64_t kmax = cdiv(nsteps, 8);        // at least 8 steps per split
  if (ks > kmax) ks = kmax;
  if (ks < 1) ks = 1;
  p.sps = cdiv(nsteps, ks);
  p.KS = cdiv(nsteps, p.sps);
  p.Mr = tiles * 64;
  if (p.KS > 1) p.part_bytes = align256(static_cast<size_t>(p.KS * p.Mr * 16 * p.nt * 4));
  return p;
}

struct WsLayout {
  size_t lora_off = 0, lora_bytes = 0;    // t or u, bf16 [M][rp]
  size_t bt_off = 0, bt_bytes = 0;        // large-M backward: B transposed, bf16 [r][N]
  size_t dp_off = 0, dp_bytes = 0;        // large M: split partials of the down-projection
  size_t total = 0;
};

// op 0: forward (lora contraction over K); op 1: backward (over N). The
// decode-shaped kernels have their own layout (counters, then split partials).
inline WsLayout ws_layout(int op, int64_t M, int64_t N, int64_t K, int r) {
  WsLayout w;
  if (M <= kSmallM) {
    w.total = op == 0 ? dec_workspace_bytes(M, 1, &N, &K) : dec_bwd_workspace_bytes(M, 1, &N, &K);
    return w;
  }
  if (r > 0) w.lora_bytes = align256(static_cast<size_t>(M * rank_pad(r) * 2));
  w.lora_off = kWsCounterBytes;
  w.bt_off = w.lora_off + w.lora_bytes;
  if (op == 1 && M > kSmallM && r > 0) w.bt_bytes = align256(static_cast<size_t>(r) * N * 2);
  w.dp_off = w.bt_off + w.bt_bytes;
  if (M > kSmallM && r > 0) w.dp_bytes = down_plan(M, op == 0 ? K : N, r).part_bytes;
  const size_t used = w.lora_bytes + w.bt_bytes + w.dp_bytes;
  w.total = used ? kWsCounterBytes + used : 0;
  return w;
}

// Adapter gradients (dA, dB): workspace plan. Mp = M rounded up to 64 (rows of
// the transposed t and u); SB / SA = row splits of the dY and x contractions.
struct GradPlan {
  int64_t Mp = 0, rp = 0, SB = 1, SA = 1;
  size_t bt_off = 0, tt_off = 0, ut_off = 0, pb_off = 0, pa_off = 0, dp_off = 0, total = 0;
};
GradPlan grad_plan(int64_t M, int64_t N, int64_t K, int r);

// qscale/step may be NULL (quantize only); otherwise the constants are also
// double-quantized in the same pass.
hipError_t launch_quantize(const void* w, int wdt, int64_t numel, uint8_t* packed, float* absmax,
                           int8_t* qscale, float* step, const Codebook& cb, hipStream_t stream);
hipError_t launch_dq_scales(const float* absmax, int64_t nblocks, int8_t* qscale, float* step,
                            hipStream_t stream);
// qscale == NULL: the constants are the fp32 absmax values (no double quantization)
hipError_t launch_dequant(const uint8_t* packed, const int8_t* qscale, const float* step, int64_t numel,
                          uint16_t* out, const Codebook& cb, hipStream_t stream, const float* absmax = nullptr);

// rank-r down projection of `in` [M][Kc] by the adapter (wrow: A [r][Kc];
// else B [Kc][r]); ldt == 0: bf16 [M][rp] (M > kSmallM); ldt > 0: bf16
// transposed, out [rp][ldt] (ldt = M rounded up to 64, rows past M zero), for
// any M.
// wt: workspace for the transposed adapter (bf16 path, wrow == false; r * Kc
// bf16); part: down_plan(M, Kc, r).part_bytes of workspace (bf16 path).
hipError_t launch_lora_down(bool wrow, const uint16_t* in, int64_t M, int64_t Kc, const uint16_t* W, int r,
                            void* out, hipStream_t stream, uint16_t* wt, float* part, int64_t ldt = 0);

// The forward of G weights, each with its own input x[i] (x[i] may repeat:
// weights that share their input). Decode shapes run launch_dec_fwd over the
// whole table; larger M runs the tiled forward per weight, reusing the
// workspace (batched_ws_bytes of it).
hipError_t launch_lora_fwd_batched(int64_t M, int G, const uint16_t* const* x, const int64_t* N, const int64_t* K,
                                   const uint8_t* const* packed, const int8_t* const* qscale,
                                   const float* const* step, const uint16_t* const* A, const uint16_t* const* B,
                                   int r, float alpha, uint16_t* const* y, void* ws, const Codebook& cb,
                                   hipStream_t stream);
size_t batched_ws_bytes(int64_t M, int G, const int64_t* N, const int64_t* K, int r);
hipError_t launch_lora_fwd(const uint16_t* x, int64_t M, int64_t N, int64_t K, const uint8_t* packed,
                           const int8_t* qscale, const float* step, const uint16_t* A, const uint16_t* B,
                           int r, float alpha, uint16_t* y, void* ws, const Codebook& cb,
                           hipStream_t stream);
hipError_t launch_bwd_dx(const uint16_t* dy, int64_t M, int64_t N, int64_t K, const uint8_t* packed,
                         const int8_t* qscale, const float* step, const uint16_t* A, const uint16_t* B,
                         int r, float alpha, uint16_t* dx, void* ws, const Codebook& cb,
                         hipStream_t stream);
// The backward dX of G independent weights: decode shapes run launch_dec_bwd
// over the whole table; larger M runs launch_bwd_dx per weight on one
// workspace (bwd_batched_ws_bytes of it).
hipError_t launch_bwd_dx_batched(int64_t M, int G, const uint16_t* const* dy, const int64_t* N, const int64_t* K,
                                 const uint8_t* const* packed, const int8_t* const* qscale,
                                 const float* const* step, const uint16_t* const* A, const uint16_t* const* B,
                                 int r, float alpha, uint16_t* const* dx, void* ws, const Codebook& cb,
                                 hipStream_t stream);
size_t bwd_batched_ws_bytes(int64_t M, int G, const int64_t* N, const int64_t* K, int r);
hipError_t launch_merge(const uint8_t* packed, const int8_t* qscale, const float* step, int64_t N, int64_t K,
                        const uint16_t* A, const uint16_t* B, int r, float alpha, uint16_t* out, const Codebook& cb,
                        hipStream_t stream);
hipError_t launch_lora_grad(const uint16_t* x, const uint16_t* dy, int64_t M, int64_t N, int64_t K,
                            const uint16_t* A, const uint16_t* B, int r, float alpha, float* dA, float* dB,
                            int accumulate, void* ws, hipStream_t stream);

// Measurement events (set through the C ABI): when set, mark_kernel(0, s)
// records the start event and mark_kernel(1, s) the stop event on stream s,
// right around the main kernel of a matmul call.
void mark_kernel(int which, hipStream_t stream);

// Built-in scratch of the allocation-free forward: a file-scope device array
// of kNoAllocScratchBytes per GPU. noalloc_scratch gives this device's address
// of it (looked up once per device, on the first call with that device
// current) after clearing its arrival counters on `stream`.
constexpr size_t kNoAllocScratchBytes = size_t{32} << 20;
hipError_t noalloc_scratch(void** ptr, hipStream_t stream);

}  // namespace qnf4
