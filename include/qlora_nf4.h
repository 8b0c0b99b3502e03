/*
 * qlora_nf4.h -- C ABI of the MI355X (gfx950) NF4 dequant-GEMM library.
 *
 * The library implements the data-parallel hot path of QLoRA as the pages
 * describe it:
 *   - block-wise 4-bit NormalFloat (NF4) quantization of a frozen weight,
 *     one 32-bit absmax constant per block of 64 weights
 *     ("A 65B fine-tune on the GPU you already have", figures 3 and 4;
 *      "QLoRA and Quantized Training", section "The idea");
 *   - double quantization of those constants to 8 bits in groups of 256
 *     blocks (same page, figure 4);
 *   - the matmul through the frozen base with the weights dequantized to
 *     bf16 block by block right before the multiply, plus the LoRA adapter
 *     term, forward and backward-to-input
 *     (same page, figure 2; "QLoRA Explained: 4-bit NF4, ...", section
 *      "What is QLoRA?"; "QLoRA and Quantized Training", section "In code").
 *
 * Storage format produced and consumed here (for a weight W of numel values,
 * nb = numel / 64 blocks, ng = ceil(nb / 256) groups):
 *   packed  uint8[numel/2]  two 4-bit codes per byte, element 2i in the low
 *                           nibble of byte i; code = index of the nearest of
 *                           the 16 levels, ties to the lower index
 *   absmax  float[nb]       per-block max |w| (the first-level constant)
 *   qscale  int8[nb]        q_b = rne(absmax_b / d_g), clamped to +-127
 *   step    float[ng]       d_g = max(absmax over group g) / 127
 * Dequantized weight: w' = bf16_rne(L[code] * fp32(q_b * d_g)).
 * The 16 levels L are the quantiles of N(0,1) at probabilities (i+1/2)/16,
 * divided by the largest one (so L[0] = -1, L[15] = +1).
 *
 * Conventions for every entry point:
 *   - bf16 tensors are passed as uint16_t bit patterns; all matrices are
 *     row-major and densely packed (leading dimension = number of columns).
 *   - Every pointer argument except those of qlora_nf4_codebook is a DEVICE
 *     pointer owned by the caller. The library never allocates or frees
 *     device memory and keeps no per-call state; it is safe to call from
 *     several threads.
 *   - `stream` is a hipStream_t (NULL = the default stream). Calls enqueue
 *     their kernels on it and return without synchronising; outputs are
 *     valid once the stream has reached them, and every buffer must stay
 *     alive until then.
 *   - Arguments are validated before anything is launched. A failed check
 *     returns a non-zero qlora_status and launches nothing. Nothing is
 *     printed and nothing aborts. A HIP launch failure returns
 *     QLORA_ERR_HIP; qlora_last_hip_error() gives the hipError_t.
 *   - Weights must be finite; NaN/Inf inputs give unspecified codes.
 */
#ifndef QLORA_NF4_H
#define QLORA_NF4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QLORA_OK = 0,
  QLORA_ERR_NULL = 1,      /* a required pointer is NULL */
  QLORA_ERR_SHAPE = 2,     /* a size is out of range or not a multiple it must be */
  QLORA_ERR_ALIGN = 3,     /* a pointer is not 16-byte aligned */
  QLORA_ERR_RANK = 4,      /* LoRA rank out of range or adapters inconsistent */
  QLORA_ERR_WORKSPACE = 5, /* workspace missing or smaller than required */
  QLORA_ERR_DTYPE = 6,     /* unknown input dtype */
  QLORA_ERR_HIP = 7,       /* a HIP call failed; see qlora_last_hip_error() */
  QLORA_ERR_INIT = 8,      /* the codebook could not be derived */
  QLORA_ERR_SCRATCH = 9    /* sizes need more than QLORA_NOALLOC_SCRATCH_BYTES */
} qlora_status;

typedef enum { QLORA_F32 = 0, QLORA_BF16 = 1 } qlora_dtype;

#define QLORA_BLOCK 64       /* weights per first-level constant */
#define QLORA_DQ_GROUP 256   /* first-level constants per second-level step */
#define QLORA_MAX_RANK 128   /* largest LoRA rank accepted */

/*
 * Block-wise NF4 quantization (figures 3 and 4 of "A 65B fine-tune on the
 * GPU you already have").
 *   w       [numel] fp32 or bf16 (wdt), the weight in any flat order (row-major
 *           [N,K] for a Linear layer); 16-byte aligned.
 *   numel   > 0, multiple of 64.
 *   packed  [numel/2] out, 16-byte aligned.
 *   absmax  [numel/64] out, per-block max |w|.
 * Codes are bit-exact functions of w: v = fp32(w / absmax) with IEEE
 * division, code = number of thresholds T_j below v, T_j the largest fp32 not
 * above the exact midpoint of levels j and j+1. An all-zero block codes 7.
 */
int qlora_nf4_quantize(const void* w, int wdt, int64_t numel, uint8_t* packed,
                       float* absmax, void* stream);

/*
 * Double quantization of the block constants to int8 in groups of 256
 * (figure 4 of "A 65B fine-tune on the GPU you already have").
 *   absmax   [nblocks] fp32 >= 0 (from qlora_nf4_quantize).
 *   nblocks  in 1 .. 2^31 - 1.
 *   qscale   [nblocks] int8 out: rne(fp32(absmax / d)), clamped to [-127, 127].
 *   step     [ceil(nblocks/256)] fp32 out: d = fp32(group max / 127); a group
 *            whose max is 0 has d = 0 and all q = 0. The last group may be
 *            partial.
 */
int qlora_dq_scales(const float* absmax, int64_t nblocks, int8_t* qscale,
                    float* step, void* stream);

/*
 * Quantize and double-quantize in one pass: the outputs of
 * qlora_nf4_quantize followed by qlora_dq_scales (bit-identical), from a
 * single kernel that handles one group of 256 blocks per workgroup.
 *   qscale [numel/64] int8 out, step [ceil(numel/16384)] fp32 out; the other
 *   arguments as in qlora_nf4_quantize.
 */
int qlora_nf4_quantize_dq(const void* w, int wdt, int64_t numel, uint8_t* packed,
                          float* absmax, int8_t* qscale, float* step,
                          void* stream);

/*
 * Standalone dequantization to bf16 (figure 2 of "A 65B fine-tune on the GPU
 * you already have"): out[i] = bf16_rne(L[code_i] * fp32(q_b * d_g)).
 *   packed [numel/2], qscale [numel/64], step [ceil(numel/16384)],
 *   numel > 0 multiple of 64, out [numel] bf16; packed and out 16-byte aligned.
 * The fused GEMMs below dequantize with exactly this arithmetic.
 */
int qlora_nf4_dequant(const uint8_t* packed, const int8_t* qscale,
                      const float* step, int64_t numel, uint16_t* out,
                      void* stream);

/*
 * Workspace (device bytes) that qlora_nf4_lora_fwd (op = 0),
 * qlora_nf4_bwd_dx (op = 1) or qlora_lora_grad (op = 2) needs for these
 * sizes; 0 when none is needed. Returns 0 for invalid sizes as well (the call
 * itself reports the error).
 *
 * Every workspace that is used at all begins with 16 KB of arrival counters
 * (the decode-shaped kernels add their split partial sums in a fixed order
 * once the last split of a tile has arrived). They must be zero when a call
 * starts, and every call leaves them zero when it completes: zero-fill a
 * workspace once after allocating it (e.g. hipMemset) and it stays valid for
 * any sequence of calls on one stream, of any entry point. Calls that run at
 * the same time need separate workspaces.
 */
size_t qlora_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, int r);

/*
 * Forward of one QLoRA linear with the dequant fused into the GEMM
 * (figure 2 of "A 65B fine-tune on the GPU you already have"; "QLoRA
 * Explained", "What is QLoRA?"; adapters r and lora_alpha as in "QLoRA and
 * Quantized Training", "In code"):
 *     y = bf16( x . W'^T + (alpha / r) . t . B^T ),  t = bf16(x . A^T)
 *   x       [M, K] bf16;  M >= 1, K multiple of 64.
 *   packed, qscale, step  the stored W [N, K] (N >= 1).
 *   A       [r, K] bf16, B [N, r] bf16 -- both NULL with r = 0 for no adapter,
 *           else 1 <= r <= 128.
 *   alpha   LoRA alpha (the update is scaled by alpha / r).
 *   y       [M, N] bf16 out.
 *   workspace / ws_bytes  device scratch of at least
 *           qlora_workspace_bytes(0, M, N, K, r) bytes, 16-byte aligned
 *           (may be NULL when that is 0). Its contents are overwritten.
 * Products are bf16 x bf16 accumulated in fp32. For M <= 16 the kernel
 * streams the weight with the contraction over K split across workgroups
 * when that fills the chip; each split then carries its part of
 * (alpha / r) . t as the sum of two bf16 values (about 16 significant bits)
 * rather than one rounding of the full t, a difference below one bf16
 * rounding of the LoRA term. x, packed, y, A, B and the
 * workspace must be 16-byte aligned. Size limits (here and in every other
 * matmul call: grouped forward, backward, merge, adapter gradients):
 * M <= 2^31, N and K <= 2^21 (each operand is addressed through 32-bit
 * buffer descriptors), and ceil(M/256) * ceil(max(N, K)/256) < 2^31 (the
 * number of 256 x 256 output tiles); larger sizes return QLORA_ERR_SHAPE.
 */
int qlora_nf4_lora_fwd(const uint16_t* x, int64_t M, int64_t N, int64_t K,
                       const uint8_t* packed, const int8_t* qscale,
                       const float* step, const uint16_t* A, const uint16_t* B,
                       int r, float alpha, uint16_t* y, void* workspace,
                       size_t ws_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the forward
 * of qlora_nf4_lora_fwd, same arguments, results and limits, but without a
 * workspace argument. The split partial sums and arrival counters live in a
 * scratch array built into the library, QLORA_NOALLOC_SCRATCH_BYTES per GPU,
 * held from the first call on that GPU until the process ends; the call
 * allocates nothing (no hipMalloc or hipFree, no host heap).
 *   Sizes whose workspace, qlora_workspace_bytes(0, M, N, K, r), exceeds
 *   QLORA_NOALLOC_SCRATCH_BYTES return QLORA_ERR_SCRATCH before any launch
 *   (the 4096 x 4096 to 22016 x 8192 layers fit at every M up to 16384 and
 *   every rank; very long K at M <= 16, or M in the hundreds of thousands,
 *   does not).
 *   Every call on one GPU shares that GPU's scratch: calls that overlap in
 *   time on one GPU (different streams or threads without ordering between
 *   them) race and give wrong results; order them on one stream. Each call
 *   first clears the counters (a small kernel on `stream`, so a captured call
 *   clears them on every replay), then runs the forward kernels.
 */
#define QLORA_NOALLOC_SCRATCH_BYTES (32u << 20)
int qlora_nf4_lora_fwd_noalloc(const uint16_t* x, int64_t M, int64_t N,
                               int64_t K, const uint8_t* packed,
                               const int8_t* qscale, const float* step,
                               const uint16_t* A, const uint16_t* B, int r,
                               float alpha, uint16_t* y, void* stream);

/*
 * Forward of several QLoRA linears that share their input (e.g. the q, k and
 * v projections of one layer), as qlora_nf4_lora_fwd on each weight i:
 *     y[i] = bf16( x . W_i'^T + (alpha / r) . (x . A_i^T) . B_i^T )
 * For M <= 16 the weights are streamed by one launch of the decode-shaped
 * kernel (qlora_nf4_lora_fwd_batched with x repeated), so the launch ramp is
 * paid once; the decode kernel chooses its split of K from the whole group,
 * so results can differ from the single calls in the fp32 summation order
 * (both within the tolerance of the single call; repeated identical calls are
 * bitwise identical). Larger M runs one LoRA down-projection per weight and
 * then one tiled GEMM launch for all G weights, whose tile order sweeps each
 * group of x rows across every weight (x is read from HBM once for the group);
 * its outputs are bitwise those of the single calls.
 *   x        [M, K] bf16 (device); G in 1..8.
 *   packed, qscale, step, N, A, B, y  host arrays of G entries: the device
 *            pointers of weight i's stored format (N[i] rows), its adapters
 *            ([r, K] and [N[i], r]; the arrays A and B may be NULL with
 *            r = 0) and its output y[i] [M, N[i]].
 *   workspace / ws_bytes  at least G * qlora_workspace_bytes(0, M, max N, K, r).
 * Alignment and size limits as in qlora_nf4_lora_fwd. Only the launch is
 * shared, not the arithmetic.
 */
int qlora_nf4_lora_fwd_grouped(const uint16_t* x, int64_t M, int64_t K, int G,
                               const uint8_t* const* packed,
                               const int8_t* const* qscale,
                               const float* const* step, const int64_t* N,
                               const uint16_t* const* A,
                               const uint16_t* const* B, int r, float alpha,
                               uint16_t* const* y, void* workspace,
                               size_t ws_bytes, void* stream);

/*
 * Forward of G independent QLoRA linears in as few launches as possible
 * (decode shapes: one launch per 32 weights, streaming all of them), e.g. the
 * linears of a model that do not depend on one another at a decode step, or
 * many small requests against different weights. For each i:
 *     y[i] = bf16( x[i] . W_i'^T + (alpha / r) . (x[i] . A_i^T) . B_i^T )
 * exactly as qlora_nf4_lora_fwd computes it ("A 65B fine-tune on the GPU you
 * already have", figure 2; "QLoRA and Quantized Training", "In code").
 *   G        1 .. QLORA_MAX_BATCH weights; M >= 1 rows for every weight.
 *   x, N, K, packed, qscale, step, A, B, y  host arrays of G entries: weight
 *            i's input x[i] [M, K[i]] bf16 (device), its shape N[i] x K[i]
 *            (each within the limits of qlora_nf4_lora_fwd), its stored
 *            format, adapters A[i] [r, K[i]], B[i] [N[i], r] (the arrays A
 *            and B may be NULL with r = 0) and its output y[i] [M, N[i]].
 *            Inputs may repeat (weights that share x).
 *   workspace / ws_bytes  at least qlora_workspace_bytes_batched(G, M, N, K,
 *            r) bytes, with the same zero-counter rule as every workspace
 *            (below).
 * M <= 16 runs the decode-shaped kernel over the whole table; larger M runs
 * the tiled forward, one GEMM launch per 8 weights (after each weight's LoRA
 * down-projection), with results bitwise those of the single calls.
 */
#define QLORA_MAX_BATCH 4096
int qlora_nf4_lora_fwd_batched(int G, int64_t M, const uint16_t* const* x,
                               const int64_t* N, const int64_t* K,
                               const uint8_t* const* packed,
                               const int8_t* const* qscale,
                               const float* const* step,
                               const uint16_t* const* A,
                               const uint16_t* const* B, int r, float alpha,
                               uint16_t* const* y, void* workspace,
                               size_t ws_bytes, void* stream);

/* Workspace bytes qlora_nf4_lora_fwd_batched needs (0 for invalid sizes). */
size_t qlora_workspace_bytes_batched(int G, int64_t M, const int64_t* N,
                                     const int64_t* K, int r);

/*
 * Backward to the input through the frozen dequantized weight (figure 2 of
 * "A 65B fine-tune on the GPU you already have": gradients flow through the
 * frozen 4-bit weights into the adapters; "QLoRA" (techbytebybyte), "Follow
 * one QLoRA training step"):
 *     dX = bf16( dY . W' + (alpha / r) . u . A ),  u = bf16(dY . B)
 *   dy      [M, N] bf16; M >= 1, N >= 1 multiple of 8, K multiple of 64.
 *   A, B, r, alpha  as in the forward; NULL/0 gives the base term only.
 *   dx      [M, K] bf16 out.
 *   workspace / ws_bytes  at least qlora_workspace_bytes(1, M, N, K, r).
 * For M <= 16 the contraction over N is split across workgroups when that
 * fills the chip, and each split carries its part of (alpha / r) . u as the
 * sum of two bf16 values (as the forward does with t at these shapes).
 */
int qlora_nf4_bwd_dx(const uint16_t* dy, int64_t M, int64_t N, int64_t K,
                     const uint8_t* packed, const int8_t* qscale,
                     const float* step, const uint16_t* A, const uint16_t* B,
                     int r, float alpha, uint16_t* dx, void* workspace,
                     size_t ws_bytes, void* stream);

/*
 * Backward dX of G independent QLoRA linears in as few launches as possible
 * (decode shapes: one launch per 32 weights, streaming all of them), e.g. the
 * linears of a model whose backward inputs are all at hand, or many small
 * requests against different weights. For each i:
 *     dx[i] = bf16( dy[i] . W_i' + (alpha / r) . u_i . A[i] ),
 *     u_i = dy[i] . B[i]
 *   dy, packed, qscale, step, N, K, A, B, dx  host arrays of G entries (G in
 *            1..QLORA_MAX_BATCH): the device pointers of weight i's operands,
 *            its sizes (N[i] >= 1 multiple of 8, K[i] multiple of 64) and its
 *            output dx[i] [M, K[i]]; one M and one rank r for all (A and B
 *            may be NULL with r = 0).
 *   workspace / ws_bytes  at least qlora_workspace_bytes_bwd_batched(G, M, N,
 *            K, r) bytes, with the zero-counter rule of every workspace.
 * M <= 16 runs the decode-shaped backward over the whole table, which carries
 * u_i as the sum of two bf16 values (about 16 significant bits) when it
 * splits a weight's rows; larger M runs the single call per weight. Results
 * equal the single calls' (within their tolerance) and repeated identical
 * calls are bitwise identical. Alignment and size limits as in
 * qlora_nf4_bwd_dx.
 */
int qlora_nf4_bwd_dx_batched(int G, int64_t M, const uint16_t* const* dy,
                             const int64_t* N, const int64_t* K,
                             const uint8_t* const* packed,
                             const int8_t* const* qscale,
                             const float* const* step,
                             const uint16_t* const* A,
                             const uint16_t* const* B, int r, float alpha,
                             uint16_t* const* dx, void* workspace,
                             size_t ws_bytes, void* stream);

/* Workspace bytes qlora_nf4_bwd_dx_batched needs (0 for invalid sizes). */
size_t qlora_workspace_bytes_bwd_batched(int G, int64_t M, const int64_t* N,
                                         const int64_t* K, int r);

/*
 * Gradients of the LoRA adapters of one QLoRA linear, the only trainable
 * parameters: the base weight is frozen and gradients and optimizer state
 * exist for the adapters alone ("QLoRA Explained", "What is QLoRA?"; "QLoRA
 * and Quantized Training", "The idea"; figure 2 of "A 65B fine-tune on the GPU
 * you already have"). They are those of the scalar <dY, y> for the forward
 * above, with s = alpha / r:
 *     dB = s . dY^T . t,  t = bf16(x . A^T)      [N, r]
 *     dA = s . u^T . x,   u = bf16(dY . B)       [r, K]
 * (t and u are the bf16 values the fused forward and backward use.)
 *   x       [M, K] bf16, the layer input of the forward; M >= 1, K multiple
 *           of 64.
 *   dy      [M, N] bf16, the gradient of y; N >= 1 multiple of 8.
 *   A, B    [r, K] and [N, r] bf16 adapters, 1 <= r <= 128; alpha as in the
 *           forward.
 *   dA, dB  [r, K] and [N, r] fp32 out (the layouts of A and B). accumulate
 *           = 0 overwrites them, 1 adds the gradients to what they hold
 *           (accumulation over micro-batches).
 *   workspace / ws_bytes  at least qlora_workspace_bytes(2, M, N, K, r).
 * Size limits as in qlora_nf4_lora_fwd.
 * Products are bf16 x bf16 accumulated in fp32; the result does not depend
 * on scheduling (partial sums are added in a fixed order). Every pointer must
 * be 16-byte aligned. The weight itself is not an argument: neither gradient
 * depends on it.
 */
int qlora_lora_grad(const uint16_t* x, const uint16_t* dy, int64_t M,
                    int64_t N, int64_t K, const uint16_t* A,
                    const uint16_t* B, int r, float alpha, float* dA,
                    float* dB, int accumulate, void* workspace,
                    size_t ws_bytes, void* stream);

/*
 * Other 16-level block formats, for comparison with NF4 ("QLoRA Explained",
 * "The three ideas behind QLoRA": NF4 beats the standard 4-bit integer and
 * float formats on normally distributed weights; figure 3 of "A 65B
 * fine-tune on the GPU you already have": uniform bins), and storage without
 * double quantization (4.5 bits per parameter, figure 4 of the same page).
 *   format  QLORA_FMT_NF4 (the levels of qlora_nf4_quantize), QLORA_FMT_INT4
 *           (the 16 evenly spaced levels (2i - 15) / 15) or QLORA_FMT_FP4 (the
 *           E2M1 values 0, 0.5, 1, 1.5, 2, 3, 4, 6 over 6, signed; -0 and +0
 *           are codes 7 and 8: v <= 0 codes -0, v > 0 codes +0); anything else
 *           gives QLORA_ERR_DTYPE.
 * Block size, absmax scaling, nearest-level rule, packing and double
 * quantization are those of the NF4 calls. qlora_q4_quantize: qscale and step
 * both NULL skips double quantization (the fp32 absmax is then the stored
 * constant), both non-NULL double-quantizes in the same pass.
 * qlora_q4_dequant: with qscale (and step) the constants are double-quantized
 * as in qlora_nf4_dequant; with qscale NULL, s = absmax[b] directly. Outputs
 * bf16 [numel]. The fused GEMMs take NF4 only.
 */
#define QLORA_FMT_NF4 0
#define QLORA_FMT_INT4 1
#define QLORA_FMT_FP4 2
int qlora_q4_quantize(const void* w, int wdt, int64_t numel, int format,
                      uint8_t* packed, float* absmax, int8_t* qscale,
                      float* step, void* stream);
int qlora_q4_dequant(const uint8_t* packed, const float* absmax,
                     const int8_t* qscale, const float* step, int64_t numel,
                     int format, uint16_t* out, void* stream);
/* Host copy of a format's 16 fp32 levels and 15 thresholds. */
int qlora_q4_codebook(int format, float levels[16], float thresholds[15]);

/*
 * Merge of the adapter into one dense bf16 weight for deployment: the LoRA
 * update is low rank and folds back into the weights ("QLoRA"
 * (techbytebybyte), "Curiosity question: is the final model permanently
 * 4-bit?", "Training setup versus deployment setup"; figure 2 of "A 65B
 * fine-tune on the GPU you already have"):
 *     out = bf16( W' + (alpha / r) . B . A )      [N, K]
 *   packed, qscale, step  the stored W [N, K]; N >= 1, K multiple of 64.
 *   A [r, K], B [N, r] bf16 (NULL with r = 0: out is exactly
 *           qlora_nf4_dequant's output); 1 <= r <= 128 otherwise.
 *   out     [N, K] bf16, 16-byte aligned.
 * W' is dequantized with the arithmetic of qlora_nf4_dequant; the rank-r sum
 * is accumulated in fp32, scaled and added to W' with one fused multiply-add,
 * then rounded to bf16 once. No workspace.
 */
int qlora_nf4_merge(const uint8_t* packed, const int8_t* qscale,
                    const float* step, int64_t N, int64_t K,
                    const uint16_t* A, const uint16_t* B, int r, float alpha,
                    uint16_t* out, void* stream);

/*
 * Host copy of the 16 fp32 levels and the 15 fp32 decision thresholds the
 * kernels use (host pointers). Derived once, in fp64, on first use.
 */
int qlora_nf4_codebook(float levels[16], float thresholds[15]);

/* Human-readable name of a qlora_status value (static storage). */
const char* qlora_status_string(int status);

/*
 * Measurement aid for profilers and benchmarks (not needed for computing):
 * while set, every matmul call records `start` (a hipEvent_t created by the
 * caller) on its stream right before launching its main kernel -- the tiled
 * GEMM, the decode-shaped kernel (the batched forward: before its first
 * launch), or the small-M backward kernel -- and `stop` right after it (after
 * the last launch), so that hipEventElapsedTime(start, stop) is that kernel's
 * duration without the LoRA down-projection or finishing launches of the same
 * call. Both NULL stops it; exactly one NULL returns QLORA_ERR_NULL. The
 * setting is process-wide: calls on other threads or streams record the same
 * events while it is set.
 */
int qlora_set_kernel_events(void* start, void* stop);

/* hipError_t of the most recent QLORA_ERR_HIP on the calling thread. */
int qlora_last_hip_error(void);

/* Library version, e.g. 1 for this ABI. */
int qlora_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_NF4_H */
