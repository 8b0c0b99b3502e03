// C ABI of the NF4 dequant-GEMM library: argument validation, codebook
// set-up and dispatch to the gfx950 kernels. Every check runs before any HIP
// call, so a rejected call launches nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/qlora_nf4.h"
#include "codebook.hpp"
#include "kernels.hpp"

namespace {

thread_local int g_last_hip_error = 0;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_status(hipError_t e) {
  if (e == hipSuccess) return QLORA_OK;
  g_last_hip_error = static_cast<int>(e);
  return QLORA_ERR_HIP;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// Shared checks of the stored weight and the adapters.
int check_weight(const uint8_t* packed, const int8_t* qscale, const float* step) {
  if (!packed || !qscale || !step) return QLORA_ERR_NULL;
  if (!aligned16(packed)) return QLORA_ERR_ALIGN;
  return QLORA_OK;
}

int check_adapter(const uint16_t* A, const uint16_t* B, int r) {
  if (r == 0) return (A == nullptr && B == nullptr) ? QLORA_OK : QLORA_ERR_RANK;
  if (r < 0 || r > QLORA_MAX_RANK) return QLORA_ERR_RANK;
  if (!A || !B) return QLORA_ERR_NULL;
  if (!aligned16(A) || !aligned16(B)) return QLORA_ERR_ALIGN;
  return QLORA_OK;
}

// Sizes of the matmul entry points. The kernels address each operand through
// 32-bit buffer descriptors whose byte range is at most 512 rows x max(N, K)
// x 2 bytes (or r x max(N, K) x 2 with r <= 128), so N and K are capped at
// 2^21; the tiled kernels number their 256 x 256 output tiles with 32-bit
// integers.
constexpr int64_t kMaxDim = int64_t{1} << 21;
constexpr int64_t kMaxM = int64_t{1} << 31;

int check_mm(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 64 || K % QLORA_BLOCK != 0) return QLORA_ERR_SHAPE;
  if (M > kMaxM || N > kMaxDim || K > kMaxDim) return QLORA_ERR_SHAPE;
  const int64_t big = N > K ? N : K;
  if (((M + 255) / 256) * ((big + 255) / 256) >= (int64_t{1} << 31)) return QLORA_ERR_SHAPE;
  return QLORA_OK;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return QLORA_OK;
  if (!ws || ws_bytes < need) return QLORA_ERR_WORKSPACE;
  if (!aligned16(ws)) return QLORA_ERR_ALIGN;
  return QLORA_OK;
}

std::atomic<void*> g_kev_start{nullptr}, g_kev_stop{nullptr};

}  // namespace

namespace qnf4 {
void mark_kernel(int which, hipStream_t stream) {
  void* e = (which == 0 ? g_kev_start : g_kev_stop).load(std::memory_order_relaxed);
  if (e) (void)hipEventRecord(static_cast<hipEvent_t>(e), stream);
}
}  // namespace qnf4

extern "C" {

int qlora_abi_version(void) { return 1; }

const char* qlora_status_string(int status) {
  switch (status) {
    case QLORA_OK: return "ok";
    case QLORA_ERR_NULL: return "null pointer";
    case QLORA_ERR_SHAPE: return "bad shape";
    case QLORA_ERR_ALIGN: return "pointer not 16-byte aligned";
    case QLORA_ERR_RANK: return "bad LoRA rank or adapters";
    case QLORA_ERR_WORKSPACE: return "workspace missing or too small";
    case QLORA_ERR_DTYPE: return "unknown dtype";
    case QLORA_ERR_HIP: return "HIP error";
    case QLORA_ERR_INIT: return "codebook derivation failed";
    case QLORA_ERR_SCRATCH: return "sizes need more than the built-in scratch of the allocation-free forward";
    default: return "unknown status";
  }
}

int qlora_last_hip_error(void) { return g_last_hip_error; }

int qlora_set_kernel_events(void* start, void* stop) {
  if ((start == nullptr) != (stop == nullptr)) return QLORA_ERR_NULL;
  g_kev_start.store(start, std::memory_order_relaxed);
  g_kev_stop.store(stop, std::memory_order_relaxed);
  return QLORA_OK;
}

int qlora_nf4_codebook(float levels[16], float thresholds[15]) {
  if (!levels || !thresholds) return QLORA_ERR_NULL;
  const qnf4::Codebook* cb = qnf4::codebook();
  if (!cb) return QLORA_ERR_INIT;
  for (int i = 0; i < 16; ++i) levels[i] = cb->L[i];
  for (int i = 0; i < 15; ++i) thresholds[i] = cb->T[i];
  return QLORA_OK;
}

size_t qlora_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, int r) {
  if (op < 0 || op > 2 || M < 1 || N < 1 || K < 64 || r < 0 || r > QLORA_MAX_RANK) return 0;
  if (op == 2) return r > 0 ? qnf4::grad_plan(M, N, K, r).total : 0;
  return qnf4::ws_layout(op, M, N, K, r).total;
}

int qlora_nf4_quantize(const void* w, int wdt, int64_t numel, uint8_t* packed, float* absmax, void* stream) {
  if (!w || !packed || !absmax) return QLORA_ERR_NULL;
  if (wdt != QLORA_F32 && wdt != QLORA_BF16) return QLORA_ERR_DTYPE;
  if (numel <= 0 || numel % QLORA_BLOCK != 0) return QLORA_ERR_SHAPE;
  if (!aligned16(w) || !aligned16(packed)) return QLORA_ERR_ALIGN;
  const qnf4::Codebook* cb = qnf4::codebook();
  if (!cb) return QLORA_ERR_INIT;
  return hip_status(qnf4::launch_quantize(w, wdt, numel, packed, absmax, nullptr, nullptr, *cb, as_stream(stream)));
}

int qlora_nf4_quantize_dq(const void* w, int wdt, int64_t numel, uint8_t* packed, float* absmax, int8_t* qscale,
                          float* step, void* stream) {
  if (!w || !packed || !absmax || !qscale || !step) return QLORA_ERR_NULL;
  if (wdt != QLORA_F32 && wdt != QLORA_BF16) return QLORA_ERR_DTYPE;
  if (numel <= 0 || numel % QLORA_BLOCK != 0) return QLORA_ERR_SHAPE;
  if (!aligned16(w) || !aligned16(packed)) return QLORA_ERR_ALIGN;
  const qnf4::Codebook* cb = qnf4::codebook();
  if (!cb) return QLORA_ERR_INIT;
  return hip_status(qnf4::launch_quantize(w, wdt, numel, packed, absmax, qscale, step, *cb, as_stream(stream)));
}

int qlora_dq_scales(const float* absmax, int64_t nblocks, int8_t* qscale, float* step, void* stream) {
  if (!absmax || !qscale || !step) return QLORA_ERR_NULL;
  if (nblocks <= 0 || nblocks >= (int64_t{1} << 31)) return QLORA_ERR_SHAPE;
  return hip_status(qnf4::launch_dq_scales(absmax, nblocks, qscale, step, as_stream(stream)));
}

int qlora_nf4_dequant(const uint8_t* packed, const int8_t* qscale, const float* step, int64_t numel,
                      uint16_t* out, void* stream) {
  int st = check_weight(packed, qscale, step);
  if (st) return st;
  if (!out) return QLORA_ERR_NULL;
  if (numel <= 0 || numel % QLORA_BLOCK != 0) return QLORA_ERR_SHAPE;
  if (!aligned16(out)) return QLORA_ERR_ALIGN;
  const qnf4::Codebook* cb = qnf4::codebook();
  if (!cb) return QLORA_ERR_INIT;
  return hip_status(qnf4::launch_dequant(packed, qscale, step, numel, out, *cb, as_stream(stream)));
}

int qlora_nf4_lora_fwd(const uint16_t* x, int64_t M, int64_t N, int64_t K, const uint8_t* packed,
                       const int8_t* qscale, const float* step, const uint16_t* A, const uint16_t* B, int r,
                       float alpha, uint16_t* y, void* workspace, size_t ws_bytes, void* stream) {
  if (!x || !y) return QLORA_ERR_NULL;
  int st = check_weight(packed, qscale, step);
  if (st) return st;
  st = check_mm(M, N, K);
  if (st) return st;
  st = check_adapter(A, B, r);
  if (st) return st;
  if (!aligned16(x) || !aligned16(y)) return QLORA_ERR_ALIGN;
  st = check_ws(workspace, ws_bytes, qnf4::ws_layout(0, M, N, K, r).total);
  if (st) return st;
  const qnf4::Codebook* cb = qnf4::codebook();
  if (!cb) return QLORA_ERR_INIT;
  return hip_status(qnf4::launch_lora_fwd(x, M, N, K, packed, qscale, step, A, B, r, alpha, y, workspace, *cb,
                                          as_stream(stream)));
}

int qlora_nf4_lora_fwd_noalloc(const uint16_t* x, int64_t M, int64_t N, int64_t K, const uint8_t* packed,
                               const int8_t* qscale, const float* step, const uint16_t* A, const uint16_t* B, int r,
                               float alpha, uint16_t* y, void* stream) {
  if (!x || !y) return QLORA_ERR_NULL;
  int st = check_weight(packed, qscale, step);
  if (st) return st;
  st = check_mm(M, N, K);
  if (st) return st;
  st = check_adapter(A, B, r);
  if (st) return st;
  if (!aligned16(x) || !aligned16(y)) return QLORA_ERR_ALIGN;
  const size_t need = qnf4::ws_layout(0, M, N, K, r).total;
  if (need > qnf4::kNoAllocScratchBytes) return QLORA_ERR_SCRATCH;
  const qnf4::Codebook* cb = qnf4::codebook();
  if (!cb) return QLORA_ERR_INIT;
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = qnf4::noalloc_scratch(&ws, as_stream(stream));
    if (e != hipSuccess) return hip_status(e);
  }
  return hip_status(
      qnf4::launch_lora_fwd(x, M, N, K, packed, qscale, step, A, B, r, alpha, y, ws, *cb, as_stream(stream)));
}

int qlora_nf4_lora_fwd_grouped(const uint16_t* x, int64_t M, int64_t K, int G, const uint8_t* const* packed,
                               const int8_t* const* qscale, const float* const* step, const int64_t* N,
                               const uint16_t* const* A, const uint16_t* const* B, int r, float alpha,
                               uint16_t* const* y, void* workspace, size_t ws_bytes, void* stream) {
  if (!x || !packed || !qscale || !step || !N || !y) return QLORA_ERR_NULL;
  if (G < 1 || G > qnf4::kMaxGroups) return QLORA_ERR_SHAPE;
  if (check_mm(M, 1, K)) return QLORA_ERR_SHAPE;
  if (r < 0 || r > QLORA_MAX_RANK) return QLORA_ERR_RANK;
  if (r > 0 && (!A || !B)) return QLORA_ERR_NULL;
  if (!aligned16(x)) return QLORA_ERR_ALIGN;
  int64_t nmax = 0;
  for (int i = 0; i < G; ++i) {
    int st = check_weight(packed[i], qscale[i], step[i]);
    if (st) return st;
    if (!y[i]) return QLORA_ERR_NULL;
    if (check_mm(M, N[i], K)) return QLORA_ERR_SHAPE;
    if (!aligned16(y[i])) return QLORA_ERR_ALIGN;
    st = check_adapter(r ? A[i] : nullptr, r ? B[i] : nullptr, r);
    if (st) return st;
    nmax = N[i] > nmax ? N[i] : nmax;
  }
  // the documented requirement, G times the single call's at the largest N,
  // is never less than what the grouped launch uses
  const size_t per = qnf4::ws_layout(0, M, nmax, K, r).total;
  const int st = check_ws(workspace, ws_bytes, per * static_cast<size_t>(G));
  if (st) return st;
  const qnf4::Codebook* cb = qnf4::codebook();
  if (!cb) return QLORA_ERR_INIT;
  const uint16_t* xs[qnf4::kMaxGroups];
  int64_t Ks[qnf4::kMaxGroups];
  for (int i = 0; i < G; ++i) {
    xs[i] = x;
    Ks[i] = K;
  }
  return hip_status(qnf4::launch_lora_fwd_batched(M, G, xs, N, Ks, packed, qscale, step, A, B, r, alpha, y,
                                                  workspace, *cb, as_stream(stream)));
}

size_t qlora_workspace_bytes_batched(int G, int64_t M, const int64_t* N, const int64_t* K, int r) {
  if (G < 1 || G > QLORA_MAX_BATCH || !N || !K || r < 0 || r > QLORA_MAX_RANK) return 0;
  for (int i = 0; i < G; ++i)
    if (check_mm(M, N[i], K[i])) return 0;
  return qnf4::batched_ws_bytes(M, G, N, K, r);
}

int qlora_nf4_lora_fwd_batched(int G, int64_t M, const uint16_t* const* x, const int64_t* N, const int64_t* K,
                               const uint8_t* const* packed, const int8_t* const* qscale,
                               const float* const* step, const uint16_t* const* A, const uint16_t* const* B,
                               int r, float alpha, uint16_t* const* y, void* workspace, size_t ws_bytes,
                               void* stream) {
  if (!x || !N || !K || !packed || !qscale || !step || !y) return QLORA_ERR_NULL;
  if (G < 1 || G > QLORA_MAX_BATCH) return QLORA_ERR_SHAPE;
  if (r < 0 || r > QLORA_MAX_RANK) return QLORA_ERR_RANK;
  if (r > 0 && (!A || !B)) return QLORA_ERR_NULL;
  for (int i = 0; i < G; ++i) {
    int st = check_weight(packed[i], qscale[i], step[i]);
    if (st) return st;
    if (!x[i] || !y[i]) return QLORA_ERR_NULL;
    if (check_mm(M, N[i], K[i])) return QLORA_ERR_SHAPE;
    if (!aligned16(x[i]) || !aligned16(y[i])) return QLORA_ERR_ALIGN;
    st = check_adapter(r ? A[i] : nullptr, r ? B[i] : nullptr, r);
    if (st) return st;
  }
  const int st = check_ws(workspace, ws_bytes, qnf4::batched_ws_bytes(M, G, N, K, r));
  if (st) return st;
  const qnf4::Codebook* cb = qnf4::codebook();
  if (!cb) return QLORA_ERR_INIT;
  return hip_status(qnf4::launch_lora_fwd_batched(M, G, x, N, K, packed, qscale, step, A, B, r, alpha, y, workspace,
                                                  *cb, as_stream(stream)));
}

int qlora_nf4_bwd_dx(const uint16_t* dy, int64_t M, int64_t N, int64_t K, const uint8_t* packed,
                     const int8_t* qscale, const float* step, const uint16_t* A, const uint16_t* B, int r,
                     float alpha, uint16_t* dx, void* workspace, size_t ws_bytes, void* stream) {
  if (!dy || !dx) return QLORA_ERR_NULL;
  int st = check_weight(packed, qscale, step);
  if (st) return st;
  if (N % 8 != 0) return QLORA_ERR_SHAPE;
  st = check_mm(M, N, K);
  if (st) return st;
  st = check_adapter(A, B, r);
  if (st) return st;
  if (!aligned16(dy) || !aligned16(dx)) return QLORA_ERR_ALIGN;
  st = check_ws(workspace, ws_bytes, qnf4::ws_layout(1, M, N, K, r).total);
  if (st) return st;
  const qnf4::Codebook* cb = qnf4::codebook();
  if (!cb) return QLORA_ERR_INIT;
  return hip_status(qnf4::launch_bwd_dx(dy, M, N, K, packed, qscale, step, A, B, r, alpha, dx, workspace, *cb,
                                        as_stream(stream)));
}

size_t qlora_workspace_bytes_bwd_batched(int G, int64_t M, const int64_t* N, const int64_t* K, int r) {
  if (G < 1 || G > QLORA_MAX_BATCH || !N || !K || r < 0 || r > QLORA_MAX_RANK) return 0;
  for (int i = 0; i < G; ++i)
    if (N[i] % 8 != 0 || check_mm(M, N[i], K[i])) return 0;
  return qnf4::bwd_batched_ws_bytes(M, G, N, K, r);
}

int qlora_nf4_bwd_dx_batched(int G, int64_t M, const uint16_t* const* dy, const int64_t* N, const int64_t* K,
                             const uint8_t* const* packed, const int8_t* const* qscale, const float* const* step,
                             const uint16_t* const* A, const uint16_t* const* B, int r, float alpha,
                             uint16_t* const* dx, void* workspace, size_t ws_bytes, void* stream) {
  if (!dy || !N || !K || !packed || !qscale || !step || !dx) return QLORA_ERR_NULL;
  if (G < 1 || G > QLORA_MAX_BATCH) return QLORA_ERR_SHAPE;
  if (r < 0 || r > QLORA_MAX_RANK) return QLORA_ERR_RANK;
  if (r > 0 && (!A || !B)) return QLORA_ERR_NULL;
  for (int i = 0; i < G; ++i) {
    int st = check_weight(packed[i], qscale[i], step[i]);
    if (st) return st;
    if (!dy[i] || !dx[i]) return QLORA_ERR_NULL;
    if (N[i] % 8 != 0 || check_mm(M, N[i], K[i])) return QLORA_ERR_SHAPE;
    if (!aligned16(dy[i]) || !aligned16(dx[i])) return QLORA_ERR_ALIGN;
    st = check_adapter(r ? A[i] : nullptr, r ? B[i] : nullptr, r);
    if (st) return st;
  }
  const int st = check_ws(workspace, ws_bytes, qnf4::bwd_batched_ws_bytes(M, G, N, K, r));
  if (st) return st;
  const qnf4::Codebook* cb = qnf4::codebook();
  if (!cb) return QLORA_ERR_INIT;
  return hip_status(qnf4::launch_bwd_dx_batched(M, G, dy, N, K, packed, qscale, step, A, B, r, alpha, dx, workspace,
                                                *cb, as_stream(stream)));
}

int qlora_q4_quantize(const void* w, int wdt, int64_t numel, int format, uint8_t* packed, float* absmax,
                      int8_t* qscale, float* step, void* stream) {
  if (!w || !packed || !absmax) return QLORA_ERR_NULL;
  if ((qscale == nullptr) != (step == nullptr)) return QLORA_ERR_NULL;
  if (wdt != QLORA_F32 && wdt != QLORA_BF16) return QLORA_ERR_DTYPE;
  if (format < 0 || format >= qnf4::kNumFormats) return QLORA_ERR_DTYPE;
  if (numel <= 0 || numel % QLORA_BLOCK != 0) return QLORA_ERR_SHAPE;
  if (!aligned16(w) || !aligned16(packed)) return QLORA_ERR_ALIGN;
  const qnf4::Codebook* cb = qnf4::codebook(format);
  if (!cb) return QLORA_ERR_INIT;
  return hip_status(qnf4::launch_quantize(w, wdt, numel, packed, absmax, qscale, step, *cb, as_stream(stream)));
}

int qlora_q4_dequant(const uint8_t* packed, const float* absmax, const int8_t* qscale, const float* step,
                     int64_t numel, int format, uint16_t* out, void* stream) {
  if (!packed || !out) return QLORA_ERR_NULL;
  if (qscale ? !step : !absmax) return QLORA_ERR_NULL;
  if (format < 0 || format >= qnf4::kNumFormats) return QLORA_ERR_DTYPE;
  if (numel <= 0 || numel % QLORA_BLOCK != 0) return QLORA_ERR_SHAPE;
  if (!aligned16(packed) || !aligned16(out)) return QLORA_ERR_ALIGN;
  const qnf4::Codebook* cb = qnf4::codebook(format);
  if (!cb) return QLORA_ERR_INIT;
  return hip_status(qnf4::launch_dequant(packed, qscale, step, numel, out, *cb, as_stream(stream),
                                         qscale ? nullptr : absmax));
}

int qlora_q4_codebook(int format, float levels[16], float thresholds[15]) {
  if (!levels || !thresholds) return QLORA_ERR_NULL;
  if (format < 0 || format >= qnf4::kNumFormats) return QLORA_ERR_DTYPE;
  const qnf4::Codebook* cb = qnf4::codebook(format);
  if (!cb) return QLORA_ERR_INIT;
  for (int i = 0; i < 16; ++i) levels[i] = cb->L[i];
  for (int i = 0; i < 15; ++i) thresholds[i] = cb->T[i];
  return QLORA_OK;
}

int qlora_nf4_merge(const uint8_t* packed, const int8_t* qscale, const float* step, int64_t N, int64_t K,
                    const uint16_t* A, const uint16_t* B, int r, float alpha, uint16_t* out, void* stream) {
  int st = check_weight(packed, qscale, step);
  if (st) return st;
  if (!out) return QLORA_ERR_NULL;
  if (check_mm(1, N, K)) return QLORA_ERR_SHAPE;
  st = check_adapter(A, B, r);
  if (st) return st;
  if (!aligned16(out)) return QLORA_ERR_ALIGN;
  const qnf4::Codebook* cb = qnf4::codebook();
  if (!cb) return QLORA_ERR_INIT;
  return hip_status(qnf4::launch_merge(packed, qscale, step, N, K, A, B, r, alpha, out, *cb, as_stream(stream)));
}

int qlora_lora_grad(const uint16_t* x, const uint16_t* dy, int64_t M, int64_t N, int64_t K, const uint16_t* A,
                    const uint16_t* B, int r, float alpha, float* dA, float* dB, int accumulate, void* workspace,
                    size_t ws_bytes, void* stream) {
  if (!x || !dy || !dA || !dB) return QLORA_ERR_NULL;
  if (N % 8 != 0 || check_mm(M, N, K)) return QLORA_ERR_SHAPE;
  if (r < 1 || r > QLORA_MAX_RANK) return QLORA_ERR_RANK;
  if (!A || !B) return QLORA_ERR_NULL;
  if (accumulate != 0 && accumulate != 1) return QLORA_ERR_SHAPE;
  if (!aligned16(x) || !aligned16(dy) || !aligned16(A) || !aligned16(B) || !aligned16(dA) || !aligned16(dB))
    return QLORA_ERR_ALIGN;
  const int st = check_ws(workspace, ws_bytes, qnf4::grad_plan(M, N, K, r).total);
  if (st) return st;
  return hip_status(qnf4::launch_lora_grad(x, dy, M, N, K, A, B, r, alpha, dA, dB, accumulate, workspace,
                                           as_stream(stream)));
}

}  // extern "C"
