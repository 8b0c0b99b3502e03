"""GPU parity of the HIP path against the CPU oracle (run on an MI355X).

Bars (stated per check):
  * codes (packed nibbles), first-level absmax, int8 scales, fp32 steps and the
    standalone dequantized bf16: bit-exact;
  * forward y and backward dX: relative Frobenius error <= 1e-2 against the
    fp64 oracle (the stated tolerance), and <= 5e-3, the bound bf16 output
    rounding (unit roundoff 2^-8) plus fp32 accumulation allows;
  * one-hot inputs (a single product per output, no adapter): bit-exact;
  * the LoRA term alone (all-zero weight): relative Frobenius <= 1e-2.
The oracle quantizes the same seeded inputs itself: nothing it is given comes
from the GPU.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import gemm, nf4

pytestmark = pytest.mark.gpu

TOL = 1e-2
TIGHT = 5e-3


@pytest.fixture(scope="module")
def qops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from qlora_dequant_gemm_amd import ops
    return ops


def dev(a):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.cuda()


def host_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def rel_fro(got, ref):
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))


def to_f64(bits):
    return gemm.bf16_to_f64(bits)


def gpu_quant(ops, w):
    qw = ops.quantize_weight(dev(w))
    return qw


# ---------------------------------------------------------------------------
# quantize / double-quant / dequant: bit-exact
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("N,K,seed", [(256, 256, 0), (3, 64, 1), (5, 192, 2), (300, 320, 3),
                                      (1000, 1024, 4)])
def test_quantize_dq_dequant_bit_exact_small(qops, N, K, seed):
    w = synth.weight(N, K, seed)
    if seed == 3:
        w[7, :64] = 0.0                           # an all-zero block
        w[9, 64:128] = -w[9, 64:128]
    packed, absmax = qops.quantize(dev(w))
    q, step = qops.dq_scales(absmax)
    torch.cuda.synchronize()
    opk, oa = nf4.quantize(w)
    oq, ostep = nf4.double_quantize(oa)
    assert np.array_equal(packed.cpu().numpy(), opk)
    assert np.array_equal(absmax.cpu().numpy().view(np.uint32), oa.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), oq)
    assert np.array_equal(step.cpu().numpy().view(np.uint32), ostep.view(np.uint32))
    qw = qops.NF4Weight(packed, q, step, (N, K))
    out = host_bits(qops.dequant(qw)).reshape(-1)
    assert np.array_equal(out, nf4.dequantize(opk, oq, ostep))


def test_quantize_bf16_input_bit_exact(qops):
    w = synth.to_bf16_bits(synth.weight(128, 512, 7))
    packed, absmax = qops.quantize(dev(w))
    opk, oa = nf4.quantize(w)
    assert np.array_equal(packed.cpu().numpy(), opk)
    assert np.array_equal(absmax.cpu().numpy(), oa)


def test_exact_level_weights_code_to_themselves(qops):
    L = nf4.codebook()
    c = np.tile(np.arange(16), 64 * 16)
    w = (L[c] * np.float32(2.0 ** -6)).astype(np.float32).reshape(64, 256)
    packed, _ = qops.quantize(dev(w))
    assert np.array_equal(nf4.unpack(packed.cpu().numpy()), c.astype(np.uint8))


def _near_threshold_weights(levels=None):
    """Blocks whose absmax is 1, so w / absmax = w exactly: every threshold,
    its fp32 neighbours and the levels themselves, in both signs."""
    levels = nf4.codebook() if levels is None else levels
    L = levels.astype(np.float64)
    vals = []
    for j in range(15):
        m = np.float32((L[j] + L[j + 1]) / 2)
        x = m
        for _ in range(3):
            x = np.nextafter(x, np.float32(-2))
        for _ in range(7):
            vals.append(x)
            x = np.nextafter(x, np.float32(2))
    vals += list(levels) + [np.float32(0.0), np.float32(-0.0), np.float32(1e-9), np.float32(-1e-9)]
    vals = np.array(vals, np.float32)
    n = 63 * ((vals.size + 62) // 63)
    vals = np.resize(vals, n).reshape(-1, 63)
    w = np.concatenate([np.ones((vals.shape[0], 1), np.float32), vals], axis=1)   # absmax 1 per block
    # the same pattern scaled by a power of two (division still exact) and by 0.37 (inexact)
    return np.concatenate([w.reshape(-1), (w * np.float32(0.125)).reshape(-1),
                           (w * np.float32(0.37)).reshape(-1)]).astype(np.float32)


@pytest.mark.parametrize("fused", [False, True])
def test_quantize_near_thresholds_bit_exact(qops, fused):
    w = _near_threshold_weights()
    w = np.concatenate([w, np.zeros(64 * 300 - w.size % (64 * 300), np.float32)]) if w.size % 64 else w
    if fused:
        packed, absmax, q, step = qops.quantize_dq(dev(w))
    else:
        packed, absmax = qops.quantize(dev(w))
        q, step = qops.dq_scales(absmax)
    opk, oa = nf4.quantize(w)
    oq, ostep = nf4.double_quantize(oa)
    assert np.array_equal(packed.cpu().numpy(), opk)
    assert np.array_equal(q.cpu().numpy(), oq)
    assert np.array_equal(step.cpu().numpy().view(np.uint32), ostep.view(np.uint32))


@pytest.mark.parametrize("N,K,bf16", [(300, 320, False), (1000, 1024, True), (3, 64, False)])
def test_fused_quantize_dq_equals_separate(qops, N, K, bf16):
    w = synth.weight(N, K, 70 + N)
    if bf16:
        w = synth.to_bf16_bits(w)
    wt = dev(w)
    p1, a1 = qops.quantize(wt)
    q1, s1 = qops.dq_scales(a1)
    p2, a2, q2, s2 = qops.quantize_dq(wt)
    for x1, x2 in [(p1, p2), (a1, a2), (q1, q2), (s1, s2)]:
        assert torch.equal(x1, x2)
    opk, oq, ostep, _ = nf4.quantize_all(w)
    assert np.array_equal(p2.cpu().numpy(), opk) and np.array_equal(q2.cpu().numpy(), oq)


@pytest.mark.parametrize("name", ["7b_attn", "7b_mlp_up"])
def test_quantize_full_size_bit_exact(qops, name):
    c = synth.CONFIGS[name]
    w = synth.weight(c["N"], c["K"], c["seeds"]["w"])
    qw = gpu_quant(qops, w)
    opk, oq, ostep, _ = nf4.quantize_all(w)
    assert np.array_equal(qw.packed.cpu().numpy(), opk)
    assert np.array_equal(qw.qscale.cpu().numpy(), oq)
    assert np.array_equal(qw.step.cpu().numpy().view(np.uint32), ostep.view(np.uint32))
    out = host_bits(qops.dequant(qw)).reshape(-1)
    assert np.array_equal(out, nf4.dequantize(opk, oq, ostep))


def test_quantize_65b_outliers_sampled_groups_bit_exact(qops):
    """65B up-projection with 0.1% x10 outliers: DQ groups are independent, so
    the oracle checks 64 random groups (and their blocks) exactly."""
    c = synth.CONFIGS["65b_up"]
    s = c["seeds"]
    w = synth.weight(c["N"], c["K"], s["w"], c["outliers"], s["outliers"])
    qw = gpu_quant(qops, w)
    packed = qw.packed.cpu().numpy()
    q = qw.qscale.cpu().numpy()
    step = qw.step.cpu().numpy()
    flat = w.reshape(-1)
    ng = step.size
    rng = np.random.Generator(np.random.PCG64(99))
    for g in sorted(rng.choice(ng, 64, replace=False)):
        lo, hi = g * 16384, (g + 1) * 16384
        opk, oa = nf4.quantize(flat[lo:hi])
        oq, ostep = nf4.double_quantize(oa)
        assert np.array_equal(packed[lo // 2:hi // 2], opk)
        assert np.array_equal(q[lo // 64:hi // 64], oq)
        assert step[g].view(np.uint32) == ostep[0].view(np.uint32)


# ---------------------------------------------------------------------------
# forward / backward, element by element at small ragged sizes
# ---------------------------------------------------------------------------
FWD_CASES = [
    # M, N, K, r, alpha, seed
    (16, 256, 256, 8, 16.0, 0),        # the tiny config
    (1, 4096 // 16, 512, 16, 32.0, 10),
    (4, 300, 320, 16, 32.0, 11),
    (5, 37, 64, 5, 7.0, 12),           # odd rank: element loads of B
    (16, 520, 768, 128, 16.0, 13),
    (17, 300, 320, 16, 32.0, 14),      # first M of the tiled path
    (300, 520, 320, 8, 16.0, 15),      # 2 x 3 tiles, ragged in M and N
    (513, 256, 128, 64, 16.0, 16),
    (260, 1, 64, 0, 0.0, 17),          # N = 1, no adapter
    (40, 136, 512, 128, 8.0, 18),      # tiled, largest rank: down-projection one round at a time
    (300, 200, 320, 96, 16.0, 19),     # tiled, six rank tiles padded to eight, ragged M and K
    (17, 64, 6144, 16, 32.0, 20),      # down-projection: three rounds per wave (the last pair half past the end)
    (4, 520, 512, 64, 16.0, 21),       # decode, four rank tiles, B rows requested during the last super-step
    (5, 300, 320, 24, 8.0, 22),        # decode, rank 24: the last 8-rank piece of each B row past r
]


def _fwd_case(ops, M, N, K, r, alpha, seed):
    w = synth.weight(N, K, seed)
    x = synth.activations(M, K, seed + 1)
    A, B = synth.adapters(N, K, r, seed + 2, seed + 3) if r else (None, None)
    qw = gpu_quant(ops, w)
    y = ops.lora_fwd(dev(x), qw, dev(A) if r else None, dev(B) if r else None, alpha)
    got = to_f64(host_bits(y))
    opk, oq, ostep, _ = nf4.quantize_all(w)
    wd = nf4.dequantize(opk, oq, ostep).reshape(N, K)
    ref = gemm.lora_forward(x, wd, A, B, alpha, r)
    return got, ref


@pytest.mark.parametrize("M,N,K,r,alpha,seed", FWD_CASES)
def test_forward_parity(qops, M, N, K, r, alpha, seed):
    got, ref = _fwd_case(qops, M, N, K, r, alpha, seed)
    e = rel_fro(got, ref)
    assert e <= TOL and e <= TIGHT, e


BWD_CASES = [
    (16, 256, 256, 8, 16.0, 20),
    (1, 64, 512, 16, 32.0, 21),
    (4, 296, 320, 16, 32.0, 22),       # N multiple of 8, not of 64
    (16, 8, 64, 4, 8.0, 23),
    (16, 1000, 768, 128, 16.0, 24),
    (17, 296, 320, 16, 32.0, 25),
    (300, 520, 320, 8, 16.0, 26),
    (513, 136, 576, 64, 16.0, 27),
    (260, 64, 64, 0, 0.0, 28),
    (5, 136, 320, 5, 7.0, 29),         # odd rank: element loads of B rows
    (3, 2000, 1024, 40, 16.0, 30),     # four rank tiles of 16; the rows split across workgroups
    (16, 4096, 64, 16, 32.0, 31),      # one block column, the rows split across workgroups
    (40, 200, 128, 32, 16.0, 32),      # B read in place, two rank tiles, a partial last chunk of N
    (33, 72, 64, 128, 8.0, 33),        # B read in place, eight rank tiles
    (40, 136, 512, 128, 8.0, 34),      # tiled: A^T of the largest rank over two full column tiles
    (300, 200, 320, 96, 16.0, 35),     # tiled: six rank tiles, ragged M and K
    (17, 6144, 64, 16, 32.0, 36),      # B read in place over three rounds per wave
]


def _bwd_case(ops, M, N, K, r, alpha, seed):
    w = synth.weight(N, K, seed)
    dy = synth.activations(M, N, seed + 1)
    A, B = synth.adapters(N, K, r, seed + 2, seed + 3) if r else (None, None)
    qw = gpu_quant(ops, w)
    dx = ops.bwd_dx(dev(dy), qw, dev(A) if r else None, dev(B) if r else None, alpha)
    got = to_f64(host_bits(dx))
    opk, oq, ostep, _ = nf4.quantize_all(w)
    wd = nf4.dequantize(opk, oq, ostep).reshape(N, K)
    ref = gemm.backward_dx(dy, wd, A, B, alpha, r)
    return got, ref


@pytest.mark.parametrize("M,N,K,r,alpha,seed", BWD_CASES)
def test_backward_parity(qops, M, N, K, r, alpha, seed):
    got, ref = _bwd_case(qops, M, N, K, r, alpha, seed)
    e = rel_fro(got, ref)
    assert e <= TOL and e <= TIGHT, e


@pytest.mark.parametrize("M,N,K", [(4, 48, 128), (16, 200, 320), (40, 300, 320), (300, 64, 576)])
def test_one_hot_forward_bit_exact(qops, M, N, K):
    """x row m = e_{k_m}: y[m, n] = W'[n, k_m], a single product per output."""
    w = synth.weight(N, K, 40 + M)
    ks = (np.arange(M) * 37 + 5) % K
    x = np.zeros((M, K), np.float32)
    x[np.arange(M), ks] = 1.0
    xb = synth.to_bf16_bits(x)
    qw = gpu_quant(qops, w)
    y = host_bits(qops.lora_fwd(dev(xb), qw))
    opk, oq, ostep, _ = nf4.quantize_all(w)
    wd = nf4.dequantize(opk, oq, ostep).reshape(N, K)
    want = wd[:, ks].T
    # -0 and +0 are the same product; compare values
    assert np.array_equal(to_f64(y), to_f64(np.ascontiguousarray(want)))


@pytest.mark.parametrize("M,N,K", [(4, 48, 128), (16, 200, 320), (40, 296, 320), (300, 64, 576)])
def test_one_hot_backward_bit_exact(qops, M, N, K):
    """dY row m = e_{n_m}: dX[m, k] = W'[n_m, k]."""
    w = synth.weight(N, K, 60 + M)
    ns = (np.arange(M) * 29 + 3) % N
    dy = np.zeros((M, N), np.float32)
    dy[np.arange(M), ns] = 1.0
    qw = gpu_quant(qops, w)
    dx = host_bits(qops.bwd_dx(dev(synth.to_bf16_bits(dy)), qw))
    opk, oq, ostep, _ = nf4.quantize_all(w)
    wd = nf4.dequantize(opk, oq, ostep).reshape(N, K)
    assert np.array_equal(to_f64(dx), to_f64(np.ascontiguousarray(wd[ns])))


@pytest.mark.parametrize("M", [4, 300])
def test_lora_term_alone(qops, M):
    """All-zero weight: every block constant is 0, so y is the LoRA term only."""
    N, K, r, alpha = 200, 320, 16, 32.0
    w = np.zeros((N, K), np.float32)
    x = synth.activations(M, K, 80)
    A, B = synth.adapters(N, K, r, 81, 82)
    qw = gpu_quant(qops, w)
    got = to_f64(host_bits(qops.lora_fwd(dev(x), qw, dev(A), dev(B), alpha)))
    ref = gemm.lora_forward(x, np.zeros((N, K), np.uint16), A, B, alpha, r)
    assert np.abs(ref).max() > 0
    assert rel_fro(got, ref) <= TOL
    dy = synth.activations(M, N, 83)
    got = to_f64(host_bits(qops.bwd_dx(dev(dy), qw, dev(A), dev(B), alpha)))
    ref = gemm.backward_dx(dy, np.zeros((N, K), np.uint16), A, B, alpha, r)
    assert rel_fro(got, ref) <= TOL


def test_determinism(qops):
    M, N, K, r = 300, 520, 320, 8
    w = synth.weight(N, K, 90)
    x = dev(synth.activations(M, K, 91))
    A, B = (dev(a) for a in synth.adapters(N, K, r, 92, 93))
    qw = gpu_quant(qops, w)
    y1 = host_bits(qops.lora_fwd(x, qw, A, B, 16.0))
    y2 = host_bits(qops.lora_fwd(x, qw, A, B, 16.0))
    assert np.array_equal(y1, y2)
    dy = dev(synth.activations(M, N, 94))
    d1 = host_bits(qops.bwd_dx(dy, qw, A, B, 16.0))
    d2 = host_bits(qops.bwd_dx(dy, qw, A, B, 16.0))
    assert np.array_equal(d1, d2)


# ---------------------------------------------------------------------------
# full-size configs: sampled outputs computed one by one by the oracle
# ---------------------------------------------------------------------------
FULL = [("7b_attn", 1), ("7b_attn", 4), ("7b_attn", 16), ("7b_mlp_up", None),
        ("7b_mlp_down", None), ("65b_up", None), ("65b_attn", None)]


@pytest.mark.parametrize("name,M", FULL)
def test_full_size_sampled(qops, name, M):
    inp = synth.config_inputs(name, M)
    M, N, K, r, alpha = inp["M"], inp["N"], inp["K"], inp["r"], inp["alpha"]
    w = inp["w"]
    qw = gpu_quant(qops, w)
    y = host_bits(qops.lora_fwd(dev(inp["x"]), qw, dev(inp["A"]), dev(inp["B"]), alpha))
    dx = host_bits(qops.bwd_dx(dev(inp["dy"]), qw, dev(inp["A"]), dev(inp["B"]), alpha))
    del qw
    torch.cuda.empty_cache()
    opk, oq, ostep, _ = nf4.quantize_all(w)
    rng = np.random.Generator(np.random.PCG64(7))
    ns = rng.integers(0, N, 64)
    ms = rng.integers(0, M, 64)
    ks = rng.integers(0, K, 64)
    rows = {int(n): nf4.dequantize_range(opk, oq, ostep, int(n) * K, (int(n) + 1) * K) for n in set(ns)}
    ref = gemm.lora_forward_at(ms, ns, inp["x"], lambda n: rows[int(n)], inp["A"], inp["B"], alpha, r)
    got = to_f64(y[ms, ns])
    assert rel_fro(got, ref) <= TIGHT
    wd = nf4.dequantize(opk, oq, ostep).reshape(N, K)
    ref = gemm.backward_dx_at(ms, ks, inp["dy"], lambda k: wd[:, int(k)], inp["A"], inp["B"], alpha, r)
    got = to_f64(dx[ms, ks])
    assert rel_fro(got, ref) <= TIGHT


# ---------------------------------------------------------------------------
# full-size configs, every output: the fused kernels against the standalone
# dequantization (bit-exact to the oracle, above) followed by an fp32 matmul,
# and bitwise repeatability. Sampling alone can miss errors confined to a few
# tiles (a stale operand in one workgroup), so every element is bounded:
#   |got - ref| <= 2^-8 |ref| + 2^-12 S + 2^-8 (alpha/r) T
# with S = sum_k |a_k||b_k| of the base product (fp32 accumulation-order
# slack) and T = sum_j |t_j||B_nj| of the adapter term (t is rounded to bf16
# on both sides; its fp32 sums may round to neighbouring bf16 values).
# ---------------------------------------------------------------------------
TILED = ["7b_mlp_up", "7b_mlp_down", "65b_up", "65b_attn"]


def _elementwise_ok(got, ref, S, T, scale):
    """Number of outputs outside the bound (NaN and Inf count as outside)."""
    bound = ref.abs() * 2.0 ** -8 + S * 2.0 ** -12 + T * (scale * 2.0 ** -8) + 1e-6
    bad = (~((got - ref).abs() <= bound)).sum().item()
    return bad


@pytest.mark.parametrize("name", TILED)
def test_full_size_every_output(qops, name):
    inp = synth.config_inputs(name, None)
    M, N, K, r, alpha = inp["M"], inp["N"], inp["K"], inp["r"], inp["alpha"]
    scale = alpha / r
    qw = gpu_quant(qops, inp["w"])
    wd = qops.dequant(qw).float()
    x, A, B = dev(inp["x"]), dev(inp["A"]), dev(inp["B"])
    y1 = qops.lora_fwd(x, qw, A, B, alpha)
    y2 = qops.lora_fwd(x, qw, A, B, alpha)
    assert torch.equal(y1, y2)
    xf, Af, Bf = x.float(), A.float(), B.float()
    t = (xf @ Af.t()).bfloat16().float()
    ref = xf @ wd.t() + scale * (t @ Bf.t())
    S = xf.abs() @ wd.abs().t()
    T = t.abs() @ Bf.abs().t()
    assert _elementwise_ok(y1.float(), ref, S, T, scale) == 0
    del y1, y2, ref, S, T, t
    dy = dev(inp["dy"])
    d1 = qops.bwd_dx(dy, qw, A, B, alpha)
    d2 = qops.bwd_dx(dy, qw, A, B, alpha)
    assert torch.equal(d1, d2)
    dyf = dy.float()
    u = (dyf @ Bf).bfloat16().float()
    ref = dyf @ wd + scale * (u @ Af)
    S = dyf.abs() @ wd.abs()
    T = u.abs() @ Af.abs()
    assert _elementwise_ok(d1.float(), ref, S, T, scale) == 0
    del qw, wd
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# the whole 7B-shaped stack, resident in HBM
# ---------------------------------------------------------------------------
def test_stack_resident_step(qops):
    """All 224 linears (32 layers x q, k, v, o, gate, up, down) quantized and
    resident together, then one step as the benchmark runs it: 224 forwards in
    layer order, 224 backward dX in reverse, outputs of equal shape sharing a
    buffer, one workspace. Checks: the resident format is the storage rate
    times the stack's parameter count (3,340,771,328 bytes); sampled DQ groups
    of every linear of layers 0 and 31 are bit-exact against the oracle; the
    outputs left by the last forward (layer 31 down) and the last backward
    (layer 0 q) match the oracle on sampled entries and equal the same calls
    made alone."""
    from oracle import storage
    L, lin, M = synth.STACK_LAYERS, synth.STACK_LINEARS, synth.STACK_M
    r, alpha = synth.STACK_R, synth.STACK_ALPHA
    lay = []
    for l in range(L):
        row = []
        for j in range(len(lin)):
            d = synth.stack_linear_device(l, j, M, acts=(l, j) in ((L - 1, 6), (0, 0)))
            d["qw"] = qops.quantize_weight(d.pop("w"))
            row.append(d)
        lay.append(row)
    params = L * sum(N * K for _, N, K in lin)
    resident = sum(d["qw"].nbytes for row in lay for d in row)
    assert params == 6_476_005_376
    assert resident == 3_340_771_328 == params * storage.bytes_per_param(1 << 16)

    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    xs = {K: torch.randn((M, K), generator=gen, device="cuda").bfloat16() for K in (4096, 11008)}
    dys = {N: torch.randn((M, N), generator=gen, device="cuda").bfloat16() for N in (4096, 11008)}
    y = {N: torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for N in (4096, 11008)}
    dx = {K: torch.empty((M, K), dtype=torch.bfloat16, device="cuda") for K in (4096, 11008)}
    ws = qops.Workspace("cuda")
    for l in range(L):
        for j, (_, N, K) in enumerate(lin):
            d = lay[l][j]
            qops.lora_fwd(d.get("x", xs[K]), d["qw"], d["A"], d["B"], alpha, out=y[N], ws=ws)
    for l in reversed(range(L)):
        for j in reversed(range(len(lin))):
            _, N, K = lin[j]
            d = lay[l][j]
            qops.bwd_dx(d.get("dy", dys[N]), d["qw"], d["A"], d["B"], alpha, out=dx[K], ws=ws)
    torch.cuda.synchronize()
    last_y, last_dx = y[4096].clone(), dx[4096].clone()
    top, bot = lay[L - 1][6], lay[0][0]
    assert torch.equal(qops.lora_fwd(top["x"], top["qw"], top["A"], top["B"], alpha), last_y)
    assert torch.equal(qops.bwd_dx(bot["dy"], bot["qw"], bot["A"], bot["B"], alpha), last_dx)

    rng = np.random.Generator(np.random.PCG64(11))
    for l in (0, L - 1):
        for j, (_, N, K) in enumerate(lin):
            w = synth.stack_linear_device(l, j, M, acts=None)["w"].cpu().numpy().reshape(-1)
            qw = lay[l][j]["qw"]
            packed, q, step = qw.packed.cpu().numpy(), qw.qscale.cpu().numpy(), qw.step.cpu().numpy()
            for g in sorted(rng.choice(step.size, 8, replace=False)):
                lo, hi = g * 16384, (g + 1) * 16384
                opk, oa = nf4.quantize(w[lo:hi])
                oq, ostep = nf4.double_quantize(oa)
                assert np.array_equal(packed[lo // 2:hi // 2], opk), (l, j, g)
                assert np.array_equal(q[lo // 64:hi // 64], oq), (l, j, g)
                assert step[g].view(np.uint32) == ostep[0].view(np.uint32), (l, j, g)

    bits = host_bits
    for d, (l, j), out, fwd in ((top, (L - 1, 6), last_y, True), (bot, (0, 0), last_dx, False)):
        _, N, K = lin[j]
        w = synth.stack_linear_device(l, j, M, acts=None)["w"].cpu().numpy()
        opk, oq, ostep, _ = nf4.quantize_all(w)
        wd = nf4.dequantize(opk, oq, ostep).reshape(N, K)
        A, B, got = bits(d["A"]), bits(d["B"]), bits(out)
        ms = rng.integers(0, M, 64)
        if fwd:
            ns = rng.integers(0, N, 64)
            ref = gemm.lora_forward_at(ms, ns, bits(d["x"]), lambda n: wd[int(n)], A, B, alpha, r)
            assert rel_fro(to_f64(got[ms, ns]), ref) <= TIGHT
        else:
            ks = rng.integers(0, K, 64)
            ref = gemm.backward_dx_at(ms, ks, bits(d["dy"]), lambda k: wd[:, int(k)], A, B, alpha, r)
            assert rel_fro(to_f64(got[ms, ks]), ref) <= TIGHT
    del lay, xs, dys, y, dx
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# adapter gradients dA, dB
# ---------------------------------------------------------------------------
GRAD_CASES = [
    # M, N, K, r, alpha, seed
    (16, 256, 256, 8, 16.0, 0),        # the tiny config
    (1, 64, 64, 16, 32.0, 1),          # a single token
    (5, 40, 64, 5, 7.0, 2),            # ragged column tile, odd rank
    (300, 520, 320, 16, 32.0, 3),      # ragged M (not a multiple of the 64-row chunk) and N
    (100, 48, 64, 32, 32.0, 4),        # two rank tiles
    (513, 264, 128, 64, 16.0, 5),      # four rank tiles
    (200, 136, 192, 128, 8.0, 6),      # the largest rank
    (4096, 1024, 512, 16, 32.0, 7),    # many row splits of two chunks each
]


def _grad_case(ops, M, N, K, r, alpha, seed):
    x = synth.activations(M, K, 400 + seed)
    dy = synth.activations(M, N, 500 + seed)
    A, B = synth.adapters(N, K, r, 600 + seed, 700 + seed)
    dA, dB = ops.lora_grad(dev(x), dev(dy), dev(A), dev(B), alpha)
    oA, oB = gemm.lora_grads(x, dy, A, B, alpha, r)
    return dA.cpu().numpy().astype(np.float64), dB.cpu().numpy().astype(np.float64), oA, oB


@pytest.mark.parametrize("M,N,K,r,alpha,seed", GRAD_CASES)
def test_adapter_grad_parity(qops, M, N, K, r, alpha, seed):
    gA, gB, oA, oB = _grad_case(qops, M, N, K, r, alpha, seed)
    assert rel_fro(gA, oA) <= TIGHT and rel_fro(gB, oB) <= TIGHT


def test_adapter_grad_accumulate_and_determinism(qops):
    M, N, K, r, alpha = 300, 520, 320, 16, 32.0
    x = dev(synth.activations(M, K, 410))
    dy = dev(synth.activations(M, N, 510))
    A, B = (dev(a) for a in synth.adapters(N, K, r, 610, 710))
    dA1, dB1 = qops.lora_grad(x, dy, A, B, alpha)
    dA2, dB2 = qops.lora_grad(x, dy, A, B, alpha)
    assert torch.equal(dA1, dA2) and torch.equal(dB1, dB2)
    # accumulate: the second call adds the same values, so the sum is exactly 2x
    qops.lora_grad(x, dy, A, B, alpha, dA=dA2, dB=dB2, accumulate=True)
    assert torch.equal(dA2, 2 * dA1) and torch.equal(dB2, 2 * dB1)
    # a stale value in the outputs is overwritten without accumulate
    dA2.fill_(float("nan"))
    dB2.fill_(float("nan"))
    qops.lora_grad(x, dy, A, B, alpha, dA=dA2, dB=dB2)
    assert torch.equal(dA1, dA2) and torch.equal(dB1, dB2)


def test_adapter_grad_rank_one_closed_form(qops):
    """One non-zero in each adapter and one-hot rows of x and dY: every output
    is a single product, so the gradients are exact."""
    M, N, K, r, alpha = 70, 72, 128, 4, 8.0
    A = np.zeros((r, K), np.float32)
    B = np.zeros((N, r), np.float32)
    A[1, 100] = 0.75
    B[9, 1] = -0.5
    x = np.zeros((M, K), np.float32)
    dy = np.zeros((M, N), np.float32)
    x[66, 100] = 1.0
    dy[66, 9] = 1.0
    bits = synth.to_bf16_bits
    dA, dB = qops.lora_grad(dev(bits(x)), dev(bits(dy)), dev(bits(A)), dev(bits(B)), alpha)
    eA = np.zeros((r, K), np.float32)
    eB = np.zeros((N, r), np.float32)
    eA[1, 100] = 2.0 * -0.5          # s * u[66, 1] * x[66, 100], u = dY . B
    eB[9, 1] = 2.0 * 0.75            # s * dY[66, 9] * t[66, 1], t = x . A^T
    assert np.array_equal(dA.cpu().numpy(), eA) and np.array_equal(dB.cpu().numpy(), eB)


@pytest.mark.parametrize("name", ["7b_mlp_up", "65b_up"])
def test_adapter_grad_full_size(qops, name):
    """Every gradient entry at full size: against the fp64 oracle (exact t, u)
    within the stated tolerance, and against an fp32 torch reference that
    rounds t and u to bf16 as the kernels do, to 1e-4."""
    inp = synth.config_inputs(name, None)
    M, N, K, r, alpha = inp["M"], inp["N"], inp["K"], inp["r"], inp["alpha"]
    x, dy, A, B = dev(inp["x"]), dev(inp["dy"]), dev(inp["A"]), dev(inp["B"])
    dA, dB = qops.lora_grad(x, dy, A, B, alpha)
    s = alpha / r
    t = (x.float() @ A.float().t()).bfloat16().float()
    u = (dy.float() @ B.float()).bfloat16().float()
    rA = s * (u.t() @ x.float())
    rB = s * (dy.float().t() @ t)
    assert (torch.linalg.norm(dA - rA) / torch.linalg.norm(rA)).item() <= 1e-4
    assert (torch.linalg.norm(dB - rB) / torch.linalg.norm(rB)).item() <= 1e-4
    gA, gB = dA.cpu().numpy().astype(np.float64), dB.cpu().numpy().astype(np.float64)
    del x, dy, A, B, dA, dB, t, u, rA, rB
    torch.cuda.empty_cache()
    oA, oB = gemm.lora_grads(inp["x"], inp["dy"], inp["A"], inp["B"], alpha, r)
    assert rel_fro(gA, oA) <= TIGHT and rel_fro(gB, oB) <= TIGHT


# ---------------------------------------------------------------------------
# merge of the adapter into one dense bf16 weight
# ---------------------------------------------------------------------------
def _merge_check(got_bits, ref, mag):
    """Every entry within one bf16 ulp of the exact fp64 value plus the fp32
    slack of the rank-r sum (2^-22 of mag = |W'| + s.|B|.|A|, which matters only
    where W' and the update cancel); returns the fraction of entries that are
    the exact value rounded to bf16 (within half an ulp)."""
    got = to_f64(got_bits)
    a = np.abs(ref)
    ulp = np.where(a > 0, np.exp2(np.floor(np.log2(np.where(a > 0, a, 1.0))) - 7), 0.0)
    assert np.all(np.abs(got - ref) <= ulp + 2.0 ** -22 * mag)
    return float(np.mean(np.abs(got - ref) <= ulp / 2))


def _merge_mag(wd, A, B, alpha, r):
    return np.abs(to_f64(wd)) + (alpha / r) * (np.abs(to_f64(B)) @ np.abs(to_f64(A)))


@pytest.mark.parametrize("N,K,r,alpha,seed", [(300, 320, 16, 32.0, 0), (37, 64, 5, 7.0, 1), (130, 1024, 64, 16.0, 2),
                                              (8, 576, 128, 8.0, 3), (200, 512, 40, 16.0, 4), (64, 256, 100, 8.0, 5)])
def test_merge_parity(qops, N, K, r, alpha, seed):
    w = synth.weight(N, K, 800 + seed)
    A, B = synth.adapters(N, K, r, 810 + seed, 820 + seed)
    qw = gpu_quant(qops, w)
    got = host_bits(qops.merge(qw, dev(A), dev(B), alpha))
    opk, oq, ostep, _ = nf4.quantize_all(w)
    wd = nf4.dequantize(opk, oq, ostep).reshape(N, K)
    assert _merge_check(got, gemm.merge(wd, A, B, alpha, r), _merge_mag(wd, A, B, alpha, r)) >= 0.99


def test_merge_without_adapter_is_dequant(qops):
    w = synth.weight(300, 320, 830)
    w[:, :64] = 0.0                                  # zero blocks dequantize to signed zeros
    qw = gpu_quant(qops, w)
    assert torch.equal(qops.merge(qw).view(torch.int16), qops.dequant(qw).view(torch.int16))


def test_merge_full_size(qops):
    inp = synth.config_inputs("7b_mlp_up", 1)
    N, K, r, alpha = inp["N"], inp["K"], inp["r"], inp["alpha"]
    qw = gpu_quant(qops, inp["w"])
    got = host_bits(qops.merge(qw, dev(inp["A"]), dev(inp["B"]), alpha))
    del qw
    torch.cuda.empty_cache()
    opk, oq, ostep, _ = nf4.quantize_all(inp["w"])
    wd = nf4.dequantize(opk, oq, ostep).reshape(N, K)
    mag = _merge_mag(wd, inp["A"], inp["B"], alpha, r)
    assert _merge_check(got, gemm.merge(wd, inp["A"], inp["B"], alpha, r), mag) >= 0.99



# ---------------------------------------------------------------------------
# other 16-level formats (INT4, FP4) and storage without double quantization
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("fmt", [1, 2])
def test_format_quantize_dequant_bit_exact(qops, fmt):
    from oracle import formats
    L = formats.levels(fmt)
    near = _near_threshold_weights(L)
    w = np.concatenate([near, np.zeros(64, np.float32),                       # and an all-zero block
                        synth.weight(300, 320, 900 + fmt).reshape(-1)])
    w = np.concatenate([w, synth.weight(1, 64 * (-(w.size // 64) % 256 + 3), 910).reshape(-1)])
    wt = dev(w)
    for dq in (True, False):
        packed, absmax, q, step = qops.q4_quantize(wt, fmt, double_quant=dq)
        opk, oa = nf4.quantize(w, L)
        assert np.array_equal(packed.cpu().numpy(), opk)
        assert np.array_equal(absmax.cpu().numpy().view(np.uint32), oa.view(np.uint32))
        if dq:
            oq, ostep = nf4.double_quantize(oa)
            assert np.array_equal(q.cpu().numpy(), oq)
            assert np.array_equal(step.cpu().numpy().view(np.uint32), ostep.view(np.uint32))
            got = host_bits(qops.q4_dequant(packed, fmt, qscale=q, step=step))
            assert np.array_equal(got, nf4.dequantize(opk, oq, ostep, levels=L))
        else:
            got = host_bits(qops.q4_dequant(packed, fmt, absmax=absmax))
            assert np.array_equal(got, nf4.dequantize(opk, None, None, levels=L, absmax=oa))


def test_format_nf4_call_equals_nf4_entry_points(qops):
    w = dev(synth.weight(256, 512, 920))
    packed, absmax, q, step = qops.q4_quantize(w, 0)
    qw = qops.quantize_weight(w)
    assert torch.equal(packed, qw.packed) and torch.equal(q, qw.qscale) and torch.equal(step, qw.step)
    assert torch.equal(qops.q4_dequant(packed, 0, qscale=q, step=step).view(torch.int16),
                       qops.dequant(qw).reshape(-1).view(torch.int16))


def test_format_error_ordering_on_7b_weight(qops):
    """The pages' claim on the 7B attention weight (N(0, 0.02)), from the GPU's
    own stored formats: NF4 has the smallest reconstruction error, with and
    without double quantization."""
    c = synth.CONFIGS["7b_attn"]
    w = dev(synth.weight(c["N"], c["K"], c["seeds"]["w"]))
    err = {}
    for fmt in (0, 1, 2):
        for dq in (True, False):
            packed, absmax, q, step = qops.q4_quantize(w, fmt, double_quant=dq)
            d = qops.q4_dequant(packed, fmt, absmax=absmax, qscale=q, step=step).float().reshape(w.shape)
            err[fmt, dq] = (torch.linalg.norm(d - w) / torch.linalg.norm(w)).item()
    print({f"{['nf4', 'int4', 'fp4'][f]}{'' if dq else '_nodq'}": round(e, 5) for (f, dq), e in err.items()})
    for dq in (True, False):
        assert err[0, dq] < err[1, dq] and err[0, dq] < err[2, dq]


# ---------------------------------------------------------------------------
# grouped forward of weights that share x
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,r", [(1, 16), (5, 0), (16, 16), (40, 16)])
def test_grouped_forward_equals_batched_and_repeats(qops, M, r):
    """The grouped forward is the batched forward with x repeated (the same
    plan, so bitwise equal), and repeated calls are bitwise identical."""
    K, Ns = 512, [512, 200, 64]
    x = dev(synth.activations(M, K, 950))
    qws, As, Bs = [], [], []
    for i, N in enumerate(Ns):
        qws.append(gpu_quant(qops, synth.weight(N, K, 960 + i)))
        A, B = synth.adapters(N, K, max(r, 1), 970 + i, 980 + i)
        As.append(dev(A) if r else None)
        Bs.append(dev(B) if r else None)
    outs = qops.lora_fwd_grouped(x, qws, As if r else None, Bs if r else None, 32.0)
    again = qops.lora_fwd_grouped(x, qws, As if r else None, Bs if r else None, 32.0)
    bat = qops.lora_fwd_batched([x] * 3, qws, As if r else None, Bs if r else None, 32.0)
    for i in range(3):
        assert torch.equal(outs[i].view(torch.int16), again[i].view(torch.int16)), i
        assert torch.equal(outs[i].view(torch.int16), bat[i].view(torch.int16)), i


def test_grouped_forward_7b_qkv(qops):
    """q, k, v of one 7B layer at M = 16 in one grouped call, each output
    against the oracle element-wise."""
    c = synth.CONFIGS["7b_attn"]
    N, K, r, alpha = c["N"], c["K"], c["r"], c["alpha"]
    x = synth.activations(16, K, 990)
    ws = [synth.weight(N, K, 991 + i) for i in range(3)]
    ad = [synth.adapters(N, K, r, 995 + i, 998 + i) for i in range(3)]
    outs = qops.lora_fwd_grouped(dev(x), [gpu_quant(qops, w) for w in ws], [dev(a) for a, _ in ad],
                                 [dev(b) for _, b in ad], alpha)
    xf = to_f64(x)
    for i in range(3):
        wd = _oracle_weight(ws[i])
        ref = gemm.lora_forward(x, wd, ad[i][0], ad[i][1], alpha, r)
        got = to_f64(host_bits(outs[i]))
        S = np.abs(xf) @ np.abs(to_f64(wd)).T
        T = np.abs(xf @ to_f64(ad[i][0]).T) @ np.abs(to_f64(ad[i][1])).T
        assert _oracle_bound_ok(got, ref, S, T, alpha / r) == 0, i


# ---------------------------------------------------------------------------
# decode shapes (M <= 16), every output against the fp64 oracle at full size.
# Same element-wise bound as the tiled kernels, with ref, S and T taken from
# the oracle's exact arithmetic (t = x . A^T and u = dY . B unrounded: the
# kernels' bf16 rounding of them is within 2^-9 s.T, inside the bound).
# The shapes cover every loop of the decode kernels: K = 4096 (the 7B
# attention projection), K = 11008 (the 7B down projection: several K steps
# per wave) and, for the backward, N = 11008 (the gate/up projections: several
# weight-row steps per slice).
# ---------------------------------------------------------------------------
def _oracle_bound_ok(got, ref, S, T, scale):
    """Number of outputs outside the bound (NaN and Inf count as outside)."""
    bound = np.abs(ref) * 2.0 ** -8 + S * 2.0 ** -12 + T * (scale * 2.0 ** -8) + 1e-6
    return int((~(np.abs(got - ref) <= bound)).sum())


def _oracle_weight(w):
    opk, oq, ostep, _ = nf4.quantize_all(w)
    return nf4.dequantize(opk, oq, ostep).reshape(w.shape)


DECODE_FWD = [("7b_attn", 1), ("7b_attn", 4), ("7b_attn", 16), ("7b_mlp_down", 1), ("7b_mlp_down", 16),
              ("7b_mlp_up", 4)]


@pytest.mark.parametrize("name,M", DECODE_FWD)
def test_decode_forward_every_output_vs_oracle(qops, name, M):
    inp = synth.config_inputs(name, M)
    N, K, r, alpha = inp["N"], inp["K"], inp["r"], inp["alpha"]
    qw = gpu_quant(qops, inp["w"])
    got = to_f64(host_bits(qops.lora_fwd(dev(inp["x"]), qw, dev(inp["A"]), dev(inp["B"]), alpha)))
    del qw
    wd = _oracle_weight(inp["w"])
    ref = gemm.lora_forward(inp["x"], wd, inp["A"], inp["B"], alpha, r)
    x, W = to_f64(inp["x"]), to_f64(wd)
    S = np.abs(x) @ np.abs(W).T
    T = np.abs(x @ to_f64(inp["A"]).T) @ np.abs(to_f64(inp["B"])).T
    assert _oracle_bound_ok(got, ref, S, T, alpha / r) == 0
    assert rel_fro(got, ref) <= TIGHT


DECODE_BWD = [("7b_attn", 16), ("7b_attn", 1), ("7b_mlp_up", 16), ("7b_mlp_up", 3), ("7b_mlp_down", 8)]


@pytest.mark.parametrize("name,M", DECODE_BWD)
def test_decode_backward_every_output_vs_oracle(qops, name, M):
    inp = synth.config_inputs(name, M)
    N, K, r, alpha = inp["N"], inp["K"], inp["r"], inp["alpha"]
    qw = gpu_quant(qops, inp["w"])
    got = to_f64(host_bits(qops.bwd_dx(dev(inp["dy"]), qw, dev(inp["A"]), dev(inp["B"]), alpha)))
    del qw
    wd = _oracle_weight(inp["w"])
    ref = gemm.backward_dx(inp["dy"], wd, inp["A"], inp["B"], alpha, r)
    dy, W = to_f64(inp["dy"]), to_f64(wd)
    S = np.abs(dy) @ np.abs(W)
    T = np.abs(dy @ to_f64(inp["B"])) @ np.abs(to_f64(inp["A"]))
    assert _oracle_bound_ok(got, ref, S, T, alpha / r) == 0
    assert rel_fro(got, ref) <= TIGHT


@pytest.mark.parametrize("M,r,Ns,K", [(1, 16, [512, 200, 64], 512), (16, 16, [4096, 4096, 4096], 4096),
                                      (4, 0, [11008, 11008], 4096), (40, 16, [300, 520], 320),
                                      (7, 32, [64, 136, 8, 1000, 72, 96, 520, 264], 768),
                                      (300, 16, [4096, 1000, 264, 8], 320), (513, 32, [520, 264, 72], 576),
                                      (257, 0, [600, 300], 1024)])
def test_grouped_forward_vs_oracle(qops, M, r, Ns, K):
    """Each output of the grouped forward against the oracle, element-wise."""
    alpha = 32.0
    x = synth.activations(M, K, 1950 + M)
    ws, As, Bs = [], [], []
    for i, N in enumerate(Ns):
        ws.append(synth.weight(N, K, 1960 + i))
        A, B = synth.adapters(N, K, max(r, 1), 1970 + i, 1980 + i)
        As.append(A)
        Bs.append(B)
    qws = [gpu_quant(qops, w) for w in ws]
    outs = qops.lora_fwd_grouped(dev(x), qws, [dev(a) for a in As] if r else None,
                                 [dev(b) for b in Bs] if r else None, alpha)
    xf = to_f64(x)
    for i, (w, out) in enumerate(zip(ws, outs)):
        wd = _oracle_weight(w)
        ref = gemm.lora_forward(x, wd, As[i], Bs[i], alpha, r)
        got = to_f64(host_bits(out))
        S = np.abs(xf) @ np.abs(to_f64(wd)).T
        T = (np.abs(xf @ to_f64(As[i]).T) @ np.abs(to_f64(Bs[i])).T) if r else np.zeros_like(S)
        assert _oracle_bound_ok(got, ref, S, T, alpha / max(r, 1)) == 0, i
        assert rel_fro(got, ref) <= TIGHT, i


def test_grouped_tiled_bitwise_equals_single_calls(qops):
    """At training shapes the grouped forward is one GEMM launch over all the
    weights; each output is bitwise the single call's (same tiles, same
    order of summation), also for a K that is not a multiple of 256."""
    for M, K, Ns in ((300, 1024, [1000, 264, 4096]), (520, 576, [520, 64])):
        r, alpha = 16, 32.0
        x = dev(synth.activations(M, K, 2100 + M))
        qws, As, Bs = [], [], []
        for i, N in enumerate(Ns):
            qws.append(gpu_quant(qops, synth.weight(N, K, 2110 + i)))
            A, B = synth.adapters(N, K, r, 2120 + i, 2130 + i)
            As.append(dev(A))
            Bs.append(dev(B))
        outs = qops.lora_fwd_grouped(x, qws, As, Bs, alpha)
        for i in range(len(Ns)):
            single = qops.lora_fwd(x, qws[i], As[i], Bs[i], alpha)
            assert np.array_equal(host_bits(outs[i]), host_bits(single)), (M, K, i)


# ---------------------------------------------------------------------------
# batched forward: independent inputs and shapes per weight in one call
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,r,G,seed", [(1, 16, 5, 0), (16, 16, 7, 1), (4, 0, 3, 2), (3, 5, 4, 3),
                                        (16, 64, 3, 4), (8, 128, 2, 5), (2, 32, 40, 6), (40, 16, 3, 7),
                                        (40, 16, 11, 8)])
def test_batched_forward_vs_oracle(qops, M, r, G, seed):
    """Weights of mixed shapes (K = 64 .. 11008, ragged N), each with its own
    x: every output against the oracle element-wise. G = 40 spans two
    launches (32 weights per launch); M = 40 takes the tiled path (one GEMM
    launch per 8 weights: G = 11 spans two)."""
    rng = np.random.Generator(np.random.PCG64(3000 + seed))
    shapes = [(int(rng.choice([8, 64, 136, 520, 1000, 4096])), int(rng.choice([64, 320, 1024, 4096, 11008])))
              for _ in range(G)]
    if G >= 3:
        shapes[0], shapes[1] = (4096, 4096), (1000, 11008)
    if G > 8:
        shapes = [(n, min(k, 1024)) for n, k in shapes]
    alpha = 16.0
    xs, ws, As, Bs = [], [], [], []
    for i, (N, K) in enumerate(shapes):
        xs.append(synth.activations(M, K, 3100 + 10 * seed + i))
        ws.append(synth.weight(N, K, 3200 + 10 * seed + i))
        A, B = synth.adapters(N, K, max(r, 1), 3300 + i, 3400 + i)
        As.append(A)
        Bs.append(B)
    outs = qops.lora_fwd_batched([dev(x) for x in xs], [gpu_quant(qops, w) for w in ws],
                                 [dev(a) for a in As] if r else None, [dev(b) for b in Bs] if r else None, alpha)
    for i, (N, K) in enumerate(shapes):
        wd = _oracle_weight(ws[i])
        ref = gemm.lora_forward(xs[i], wd, As[i], Bs[i], alpha, r)
        got = to_f64(host_bits(outs[i]))
        xf = to_f64(xs[i])
        S = np.abs(xf) @ np.abs(to_f64(wd)).T
        T = (np.abs(xf @ to_f64(As[i]).T) @ np.abs(to_f64(Bs[i])).T) if r else np.zeros_like(S)
        assert _oracle_bound_ok(got, ref, S, T, alpha / max(r, 1)) == 0, (i, N, K)


# ---------------------------------------------------------------------------
# batched backward: independent dY and shapes per weight in one call
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,r,G,seed", [(1, 16, 5, 0), (16, 16, 7, 1), (4, 0, 3, 2), (3, 5, 4, 3),
                                        (16, 64, 3, 4), (2, 32, 40, 6), (40, 16, 3, 7)])
def test_batched_backward_vs_oracle(qops, M, r, G, seed):
    """Weights of mixed shapes (K = 64 .. 11008, N a multiple of 8 up to
    11008), each with its own dY: every output against the oracle
    element-wise. G = 40 spans two launches (32 weights per launch); M = 40
    takes the tiled path (one call per weight)."""
    rng = np.random.Generator(np.random.PCG64(3700 + seed))
    shapes = [(int(rng.choice([8, 64, 136, 520, 1000, 4096])), int(rng.choice([64, 320, 1024, 4096, 11008])))
              for _ in range(G)]
    if G >= 3:
        shapes[0], shapes[1] = (4096, 4096), (11008, 1024)
    if G > 8:
        shapes = [(n, min(k, 1024)) for n, k in shapes]
    alpha = 16.0
    dys, ws, As, Bs = [], [], [], []
    for i, (N, K) in enumerate(shapes):
        dys.append(synth.activations(M, N, 3800 + 10 * seed + i))
        ws.append(synth.weight(N, K, 3900 + 10 * seed + i))
        A, B = synth.adapters(N, K, max(r, 1), 4000 + i, 4100 + i)
        As.append(A)
        Bs.append(B)
    outs = qops.bwd_dx_batched([dev(d) for d in dys], [gpu_quant(qops, w) for w in ws],
                               [dev(a) for a in As] if r else None, [dev(b) for b in Bs] if r else None, alpha)
    for i, (N, K) in enumerate(shapes):
        wd = _oracle_weight(ws[i])
        ref = gemm.backward_dx(dys[i], wd, As[i], Bs[i], alpha, r)
        got = to_f64(host_bits(outs[i]))
        df = to_f64(dys[i])
        S = np.abs(df) @ np.abs(to_f64(wd))
        T = (np.abs(df @ to_f64(Bs[i])) @ np.abs(to_f64(As[i]))) if r else np.zeros_like(S)
        assert _oracle_bound_ok(got, ref, S, T, alpha / max(r, 1)) == 0, (i, N, K)


@pytest.mark.parametrize("M,r,K,seed", [(16, 16, 4096, 0), (3, 5, 4032, 1), (1, 32, 4096, 2), (8, 0, 4032, 3)])
def test_batched_backward_wide_items_vs_oracle(qops, M, r, K, seed):
    """Eight weights sharing K (128 or more 256-column ranges in the launch,
    so the backward runs its 256-column items; K = 4032 leaves a ragged last
    range): every output against the oracle element-wise."""
    Ns = [4096, 2000, 520, 8, 11008, 4096, 1000, 64]
    alpha = 16.0
    dys, ws, As, Bs = [], [], [], []
    for i, N in enumerate(Ns):
        dys.append(synth.activations(M, N, 4600 + 10 * seed + i))
        ws.append(synth.weight(N, K, 4700 + 10 * seed + i))
        A, B = synth.adapters(N, K, max(r, 1), 4800 + i, 4900 + i)
        As.append(A)
        Bs.append(B)
    outs = qops.bwd_dx_batched([dev(d) for d in dys], [gpu_quant(qops, w) for w in ws],
                               [dev(a) for a in As] if r else None, [dev(b) for b in Bs] if r else None, alpha)
    for i, N in enumerate(Ns):
        wd = _oracle_weight(ws[i])
        ref = gemm.backward_dx(dys[i], wd, As[i], Bs[i], alpha, r)
        got = to_f64(host_bits(outs[i]))
        df = to_f64(dys[i])
        S = np.abs(df) @ np.abs(to_f64(wd))
        T = (np.abs(df @ to_f64(Bs[i])) @ np.abs(to_f64(As[i]))) if r else np.zeros_like(S)
        assert _oracle_bound_ok(got, ref, S, T, alpha / max(r, 1)) == 0, (i, N, K)


def test_batched_backward_repeats_bitwise(qops):
    """Repeated identical batched calls through one workspace are bitwise
    identical and leave its arrival counters zero."""
    M, r = 16, 16
    shapes = [(4096, 1024), (11008, 64), (520, 320)]
    dys = [dev(synth.activations(M, N, 4200 + i)) for i, (N, K) in enumerate(shapes)]
    qws = [gpu_quant(qops, synth.weight(N, K, 4300 + i)) for i, (N, K) in enumerate(shapes)]
    ad = [synth.adapters(N, K, r, 4400 + i, 4500 + i) for i, (N, K) in enumerate(shapes)]
    As, Bs = [dev(a) for a, _ in ad], [dev(b) for _, b in ad]
    ws = qops.Workspace("cuda")
    o1 = qops.bwd_dx_batched(dys, qws, As, Bs, 32.0, ws=ws)
    torch.cuda.synchronize()
    assert int(ws.buf[:16384].view(torch.int32).abs().sum()) == 0
    o2 = qops.bwd_dx_batched(dys, qws, As, Bs, 32.0, ws=ws)
    for a, b in zip(o1, o2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_decode_split_fixup_counters_left_zero(qops):
    """A call whose K is split across workgroups leaves the workspace's arrival
    counters zero, so the same workspace serves any later call; repeated calls
    through one workspace are bitwise identical."""
    M, N, K, r = 16, 1000, 11008, 16
    x = dev(synth.activations(M, K, 3500))
    qw = gpu_quant(qops, synth.weight(N, K, 3501))
    A, B = (dev(a) for a in synth.adapters(N, K, r, 3502, 3503))
    ws = qops.Workspace("cuda")
    assert qops.workspace_bytes(0, M, N, K, r) > 16384
    y1 = qops.lora_fwd(x, qw, A, B, 32.0, ws=ws)
    torch.cuda.synchronize()
    assert int(ws.buf[:16384].view(torch.int32).abs().sum()) == 0
    y2 = qops.lora_fwd(x, qw, A, B, 32.0, ws=ws)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_decode_bwd_split_fixup_counters_left_zero(qops):
    """A decode-shaped backward whose rows are split across workgroups leaves
    the workspace's arrival counters zero; repeated calls through one
    workspace are bitwise identical."""
    M, N, K, r = 16, 11008, 1024, 16
    dy = dev(synth.activations(M, N, 3600))
    qw = gpu_quant(qops, synth.weight(N, K, 3601))
    A, B = (dev(a) for a in synth.adapters(N, K, r, 3602, 3603))
    ws = qops.Workspace("cuda")
    assert qops.workspace_bytes(1, M, N, K, r) > 16384
    d1 = qops.bwd_dx(dy, qw, A, B, 32.0, ws=ws)
    torch.cuda.synchronize()
    assert int(ws.buf[:16384].view(torch.int32).abs().sum()) == 0
    d2 = qops.bwd_dx(dy, qw, A, B, 32.0, ws=ws)
    assert torch.equal(d1.view(torch.int16), d2.view(torch.int16))
