"""Forward and backward of one QLoRA linear layer, fp64 -- oracle.

TEST INFRASTRUCTURE (see the package docstring).

Sources, cited by page title and section:
  [ARCH-fig2] "A 65B fine-tune on the GPU you already have", figure 2 (the
              architecture): the frozen weights are dequantized to bf16 for
              the multiply, gradients flow through them into the adapters, and
              the LoRA low-rank update is the usual one.
  [WHAT]      "QLoRA Explained: ...", section "What is QLoRA?": 4-bit base
              dequantized to a 16-bit compute type for each matrix multiply;
              only the adapters carry gradients.
  [CODE]      "QLoRA and Quantized Training", section "In code": adapter rank
              r and lora_alpha; section "The idea": adapters kept in bf16.
  [STEP]      "QLoRA" (techbytebybyte), section "Follow one QLoRA training
              step": gradients go into the adapters, not the frozen base.

  [MERGE]     "QLoRA" (techbytebybyte), "Curiosity question: is the final
              model permanently 4-bit?", "Training setup versus deployment
              setup" and "Common misconception" (the adapter can be merged
              back into the weights for deployment); "A 65B fine-tune on the
              GPU you already have", figure 2 (same low-rank update, same
              mergeability).
  [BASE]      "QLoRA Explained: ...", "What is QLoRA?" (the base is frozen:
              gradients and optimizer state exist only for the adapters);
              "QLoRA and Quantized Training", "The idea" (the adapters hold
              the gradients and optimizer state, in bf16).

Definitions (the LoRA scale alpha/r is the standard one for these knobs):
  forward   y  = x . W'^T + (alpha/r) . (x . A^T) . B^T
  backward  dX = dY . W'  [+ (alpha/r) . (dY . B) . A]
  adapters  dB = (alpha/r) . dY^T . (x . A^T)      [N, r]
            dA = (alpha/r) . (dY . B)^T . x        [r, K]
  merge     W'' = W' + (alpha/r) . B . A             [N, K]
with W' [N,K] the dequantized bf16 weight, x [M,K], A [r,K], B [N,r],
dY [M,N]. The adapter gradients are those of the scalar <dY, y> with respect
to B and A: y is linear in each adapter with the other held fixed. Inputs are bf16 bit patterns (uint16); the products are taken in
fp64 on the exact bf16 values, which is the real-number result the bf16
kernels approximate. r == 0 means no adapter.
"""
import numpy as np


def bf16_to_f64(bits):
    """Exact value of bf16 bit patterns, as fp64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def lora_forward(x_bits, wdeq_bits, A_bits=None, B_bits=None, alpha=0.0, r=0):
    """y [M,N] in fp64 ([ARCH-fig2], [WHAT], [CODE])."""
    x = bf16_to_f64(x_bits)
    W = bf16_to_f64(wdeq_bits)
    y = x @ W.T
    if r:
        A = bf16_to_f64(A_bits)
        B = bf16_to_f64(B_bits)
        y = y + (alpha / r) * ((x @ A.T) @ B.T)
    return y


def backward_dx(dy_bits, wdeq_bits, A_bits=None, B_bits=None, alpha=0.0, r=0):
    """dX [M,K] in fp64 ([ARCH-fig2], [STEP])."""
    dy = bf16_to_f64(dy_bits)
    W = bf16_to_f64(wdeq_bits)
    dx = dy @ W
    if r:
        A = bf16_to_f64(A_bits)
        B = bf16_to_f64(B_bits)
        dx = dx + (alpha / r) * ((dy @ B) @ A)
    return dx


def lora_forward_at(ms, ns, x_bits, wrow, A_bits=None, B_bits=None, alpha=0.0, r=0):
    """y[ms[i], ns[i]] for sampled index pairs, fp64.

    ``wrow(n)`` returns the dequantized bf16 row n of W' (uint16[K]); only the
    sampled rows are materialised, so this works at full model sizes.
    """
    x = bf16_to_f64(x_bits)
    out = np.empty(len(ms), dtype=np.float64)
    if r:
        A = bf16_to_f64(A_bits)
        B = bf16_to_f64(B_bits)
    for i, (m, n) in enumerate(zip(ms, ns)):
        acc = float(np.dot(x[m], bf16_to_f64(wrow(n))))
        if r:
            acc += (alpha / r) * float(np.dot(x[m] @ A.T, B[n]))
        out[i] = acc
    return out


def backward_dx_at(ms, ks, dy_bits, wcol, A_bits=None, B_bits=None, alpha=0.0, r=0):
    """dX[ms[i], ks[i]] for sampled index pairs, fp64.

    ``wcol(k)`` returns column k of W' (uint16[N]).
    """
    dy = bf16_to_f64(dy_bits)
    out = np.empty(len(ms), dtype=np.float64)
    if r:
        A = bf16_to_f64(A_bits)
        B = bf16_to_f64(B_bits)
    for i, (m, k) in enumerate(zip(ms, ks)):
        acc = float(np.dot(dy[m], bf16_to_f64(wcol(k))))
        if r:
            acc += (alpha / r) * float(np.dot(dy[m] @ B, A[:, k]))
        out[i] = acc
    return out


def lora_grads(x_bits, dy_bits, A_bits, B_bits, alpha, r):
    """(dA [r,K], dB [N,r]) in fp64 ([ARCH-fig2], [STEP], [BASE]).

    With s = alpha/r, t = x . A^T and u = dY . B (exact, no rounding):
    dB = s . dY^T . t and dA = s . u^T . x.
    """
    x = bf16_to_f64(x_bits)
    dy = bf16_to_f64(dy_bits)
    A = bf16_to_f64(A_bits)
    B = bf16_to_f64(B_bits)
    s = alpha / r
    t = x @ A.T
    u = dy @ B
    return s * (u.T @ x), s * (dy.T @ t)


def merge(wdeq_bits, A_bits=None, B_bits=None, alpha=0.0, r=0):
    """W' + (alpha/r) . B . A [N,K] in fp64 ([MERGE], [ARCH-fig2]): the one
    dense weight whose forward equals the adapted layer's, x . W''^T =
    x . W'^T + (alpha/r) . (x . A^T) . B^T."""
    W = bf16_to_f64(wdeq_bits)
    if not r:
        return W
    return W + (alpha / r) * (bf16_to_f64(B_bits) @ bf16_to_f64(A_bits))
