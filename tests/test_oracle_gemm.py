"""Pins of the oracle's forward and backward of one QLoRA linear.

Sources: "A 65B fine-tune on the GPU you already have", figure 2 (bf16
dequant before the multiply; gradients flow through the frozen weights into
the adapters; the usual LoRA low-rank update); "QLoRA and Quantized
Training", "In code" (r, lora_alpha).

Pins used: one-hot inputs (a single product per output), the adjoint identity
<fwd(x), dY> = <x, bwd(dY)> that fixes every transposition, a closed-form
rank-one adapter, linearity, and a pure-Python scalar loop on a tiny case.
Adapter gradients: directional derivatives taken through the forward itself
(y is linear in each adapter), torch autograd in fp64, and a one-hot closed
form.
"""
import math

import numpy as np

from oracle import gemm, nf4
import synth


def _setup(M, N, K, r, seed):
    w = synth.weight(N, K, seed)
    packed, q, step, _ = nf4.quantize_all(w)
    wd = nf4.dequantize(packed, q, step).reshape(N, K)
    x = synth.activations(M, K, seed + 1)
    A, B = synth.adapters(N, K, r, seed + 2, seed + 3) if r else (None, None)
    dy = synth.activations(M, N, seed + 4)
    return wd, x, A, B, dy


def _bits(a):
    return synth.to_bf16_bits(np.asarray(a, dtype=np.float32))


def test_one_hot_rows_pick_weight_columns():
    N, K = 48, 128
    wd, *_ = _setup(1, N, K, 0, 50)
    ks = [0, 5, 64, 127]
    x = np.zeros((len(ks), K), np.float32)
    for m, k in enumerate(ks):
        x[m, k] = 1.0
    y = gemm.lora_forward(_bits(x), wd)
    W = nf4.bf16_bits_to_f32(wd).astype(np.float64)
    for m, k in enumerate(ks):
        assert np.array_equal(y[m], W[:, k])
    dy = np.zeros((2, N), np.float32)
    dy[0, 3] = 1.0
    dy[1, 47] = 1.0
    dx = gemm.backward_dx(_bits(dy), wd)
    assert np.array_equal(dx[0], W[3]) and np.array_equal(dx[1], W[47])


def test_adjoint_identity_base_and_lora():
    """sum(y * dY) == sum(x * dX) for y = f(x), dX = f^T(dY), term by term."""
    M, N, K, r = 7, 40, 192, 4
    wd, x, A, B, dy = _setup(M, N, K, r, 60)
    xf = gemm.bf16_to_f64(x)
    dyf = gemm.bf16_to_f64(dy)
    for args in [(None, None, 0.0, 0), (A, B, 3.0, r)]:
        y = gemm.lora_forward(x, wd, *args)
        dx = gemm.backward_dx(dy, wd, *args)
        lhs, rhs = np.sum(y * dyf), np.sum(xf * dx)
        assert abs(lhs - rhs) <= 1e-9 * (np.abs(y * dyf).sum() + 1)


def test_rank_one_adapter_closed_form():
    """A has one non-zero A[j,k]=a, B one non-zero B[n,j]=b: the LoRA term is
    (alpha/r)*a*b*x[:,k] in column n and zero elsewhere."""
    M, N, K, r = 5, 16, 64, 4
    x = synth.activations(M, K, 70)
    zero_w = np.zeros(N * K, np.uint16).reshape(N, K)
    A = np.zeros((r, K), np.float32)
    B = np.zeros((N, r), np.float32)
    A[2, 9] = 0.5
    B[11, 2] = -0.25
    y = gemm.lora_forward(x, zero_w, _bits(A), _bits(B), alpha=8.0, r=r)
    expect = np.zeros((M, N))
    expect[:, 11] = (8.0 / r) * 0.5 * -0.25 * gemm.bf16_to_f64(x)[:, 9]
    assert np.array_equal(y, expect)


def test_linearity_and_alpha_scaling():
    M, N, K, r = 6, 32, 128, 8
    wd, x, A, B, _ = _setup(M, N, K, r, 80)
    base = gemm.lora_forward(x, wd)
    y1 = gemm.lora_forward(x, wd, A, B, 16.0, r)
    y2 = gemm.lora_forward(x, wd, A, B, 32.0, r)
    assert np.allclose(y2 - base, 2 * (y1 - base), rtol=1e-12, atol=1e-15)


def test_scalar_loop_reference_tiny():
    """Pure-Python math.fsum loops, indices written out, on a tiny case."""
    M, N, K, r = 2, 3, 64, 2
    wd, x, A, B, dy = _setup(M, N, K, r, 90)
    f = lambda b: float(gemm.bf16_to_f64(np.array([b], np.uint16))[0])
    alpha = 6.0
    y = gemm.lora_forward(x, wd, A, B, alpha, r)
    dx = gemm.backward_dx(dy, wd, A, B, alpha, r)
    for m in range(M):
        t = [math.fsum(f(x[m, k]) * f(A[j, k]) for k in range(K)) for j in range(r)]
        for n in range(N):
            base = math.fsum(f(x[m, k]) * f(wd[n, k]) for k in range(K))
            lora = math.fsum(t[j] * f(B[n, j]) for j in range(r))
            assert abs(y[m, n] - (base + alpha / r * lora)) < 1e-12
        u = [math.fsum(f(dy[m, n]) * f(B[n, j]) for n in range(N)) for j in range(r)]
        for k in range(K):
            base = math.fsum(f(dy[m, n]) * f(wd[n, k]) for n in range(N))
            lora = math.fsum(u[j] * f(A[j, k]) for j in range(r))
            assert abs(dx[m, k] - (base + alpha / r * lora)) < 1e-12


def test_sampled_entries_equal_full_products():
    M, N, K, r = 9, 70, 256, 8
    wd, x, A, B, dy = _setup(M, N, K, r, 95)
    y = gemm.lora_forward(x, wd, A, B, 4.0, r)
    dx = gemm.backward_dx(dy, wd, A, B, 4.0, r)
    rng = np.random.Generator(np.random.PCG64(1))
    ms = rng.integers(0, M, 40)
    ns = rng.integers(0, N, 40)
    ks = rng.integers(0, K, 40)
    ys = gemm.lora_forward_at(ms, ns, x, lambda n: wd[n], A, B, 4.0, r)
    ds = gemm.backward_dx_at(ms, ks, dy, lambda k: wd[:, k], A, B, 4.0, r)
    assert np.allclose(ys, y[ms, ns], rtol=1e-12, atol=1e-12)
    assert np.allclose(ds, dx[ms, ks], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# adapter gradients dA, dB (the gradients of <dY, y> with respect to A and B)
# ---------------------------------------------------------------------------
def test_adapter_grads_directional_derivatives_through_forward():
    """y is linear in B with A fixed and in A with B fixed, so for any
    direction E of B and F of A the forward itself (weight zero) gives
    <dY, fwd(x; A, E)> = <dB, E> and <dY, fwd(x; F, B)> = <dA, F>. Shapes
    are all distinct, so a transposed or swapped gradient cannot pass."""
    M, N, K, r = 9, 40, 192, 5
    _, x, A, B, dy = _setup(M, N, K, r, 300)
    alpha = 7.0
    dA, dB = gemm.lora_grads(x, dy, A, B, alpha, r)
    assert dA.shape == (r, K) and dB.shape == (N, r)
    zero_n = np.zeros((N, K), np.uint16)
    dyf = gemm.bf16_to_f64(dy)
    rng = np.random.Generator(np.random.PCG64(301))
    for _ in range(3):
        E = _bits(rng.standard_normal((N, r)).astype(np.float32))
        F = _bits(rng.standard_normal((r, K)).astype(np.float32))
        lb = np.sum(dyf * gemm.lora_forward(x, zero_n, A, E, alpha, r))
        la = np.sum(dyf * gemm.lora_forward(x, zero_n, F, B, alpha, r))
        ib = np.sum(dB * gemm.bf16_to_f64(E))
        ia = np.sum(dA * gemm.bf16_to_f64(F))
        assert abs(lb - ib) <= 1e-10 * (abs(lb) + 1)
        assert abs(la - ia) <= 1e-10 * (abs(la) + 1)


def test_adapter_grads_match_autograd():
    """torch autograd (CPU, fp64) of <dY, x W'^T + s (x A^T) B^T> with respect to
    A and B: an independent derivation of the same gradients."""
    import torch
    M, N, K, r = 13, 24, 128, 8
    wd, x, A, B, dy = _setup(M, N, K, r, 310)
    alpha = 16.0
    dA, dB = gemm.lora_grads(x, dy, A, B, alpha, r)
    T = lambda a: torch.from_numpy(gemm.bf16_to_f64(a))
    xt, wt, dyt = T(x), T(wd), T(dy)
    At, Bt = T(A).requires_grad_(), T(B).requires_grad_()
    y = xt @ wt.T + (alpha / r) * (xt @ At.T) @ Bt.T
    (y * dyt).sum().backward()
    assert np.allclose(dA, At.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dB, Bt.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_adapter_grads_one_hot_closed_form():
    """x = e_k in row m, dY = e_n in row m: dB[n, :] = s A[:, k] and
    dA[:, k] = s B[n, :], everything else zero (single products, exact)."""
    M, N, K, r = 3, 16, 64, 4
    _, _, A, B, _ = _setup(1, N, K, r, 320)
    x = np.zeros((M, K), np.float32)
    dy = np.zeros((M, N), np.float32)
    x[1, 37] = 1.0
    dy[1, 5] = 1.0
    dA, dB = gemm.lora_grads(_bits(x), _bits(dy), A, B, 8.0, r)
    eA = np.zeros((r, K))
    eB = np.zeros((N, r))
    eB[5] = 2.0 * gemm.bf16_to_f64(A)[:, 37]
    eA[:, 37] = 2.0 * gemm.bf16_to_f64(B)[5]
    assert np.array_equal(dA, eA) and np.array_equal(dB, eB)


# ---------------------------------------------------------------------------
# merge of the adapter into one dense weight
# ---------------------------------------------------------------------------
def test_merge_forward_equals_adapted_forward():
    """x . W''^T == x . W'^T + s . (x . A^T) . B^T (associativity), on a
    non-square shape so that a transposed or swapped product cannot pass."""
    M, N, K, r = 7, 40, 192, 5
    wd, x, A, B, _ = _setup(M, N, K, r, 330)
    merged = gemm.merge(wd, A, B, 6.0, r)
    assert merged.shape == (N, K)
    lhs = gemm.bf16_to_f64(x) @ merged.T
    rhs = gemm.lora_forward(x, wd, A, B, 6.0, r)
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def test_merge_without_adapter_and_rank_one():
    N, K, r = 16, 64, 4
    wd, _, _, _, _ = _setup(1, N, K, 0, 340)
    assert np.array_equal(gemm.merge(wd), gemm.bf16_to_f64(wd))
    A = np.zeros((r, K), np.float32)
    B = np.zeros((N, r), np.float32)
    A[3, 10] = 0.25
    B[7, 3] = 2.0
    m = gemm.merge(np.zeros((N, K), np.uint16), _bits(A), _bits(B), 8.0, r)
    e = np.zeros((N, K))
    e[7, 10] = 2.0 * 0.25 * 2.0
    assert np.array_equal(m, e)
