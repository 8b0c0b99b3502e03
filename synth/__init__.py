"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random numbers and shapes them; it holds none of the
quantization or matmul arithmetic, so both the HIP path and the CPU oracle can
consume its outputs without sharing any of the method's code.

Workloads follow the shapes the pages talk about (a 7B-class model's attention
and MLP projections; a 65B-class layer) and the recipe below:
  * frozen weights W [N, K] fp32 ~ N(0, 0.02) (0.02 is the standard deviation);
  * the 65B-shaped layers add round(0.001 * numel) outliers (distinct flat
    indices, chosen without replacement) multiplied by 10;
  * activations x and upstream gradients dY ~ N(0, 1), drawn in fp32 and
    rounded to bf16 (round to nearest even, by torch's CPU conversion);
  * LoRA adapters A [r, K] and B [N, r] ~ N(0, 0.01), rounded to bf16.
bf16 arrays are returned as uint16 bit patterns.
"""
import numpy as np

WEIGHT_STD = 0.02
ADAPTER_STD = 0.01

# name -> shape, adapter and seed table. Seeds: w, x, A, B, dY (+ outliers).
CONFIGS = {
    "tiny": dict(N=256, K=256, M=(16,), r=8, alpha=16.0,
                 seeds=dict(w=0, x=1, A=2, B=3, dy=4)),
    "7b_attn": dict(N=4096, K=4096, M=(1, 4, 16), r=16, alpha=32.0,
                    seeds=dict(w=10, x=11, A=12, B=13, dy=14)),
    "7b_mlp_up": dict(N=11008, K=4096, M=(4096,), r=16, alpha=32.0,
                      seeds=dict(w=20, x=21, A=22, B=23, dy=24)),
    "7b_mlp_down": dict(N=4096, K=11008, M=(4096,), r=16, alpha=32.0,
                        seeds=dict(w=25, x=26, A=27, B=28, dy=29)),
    "65b_up": dict(N=22016, K=8192, M=(2048,), r=64, alpha=16.0, outliers=0.001,
                   seeds=dict(w=30, x=31, A=32, B=33, dy=34, outliers=35)),
    "65b_attn": dict(N=8192, K=8192, M=(2048,), r=64, alpha=16.0, outliers=0.001,
                     seeds=dict(w=36, x=37, A=38, B=39, dy=40, outliers=41)),
}

# The 7B-shaped stack: 32 layers of q, k, v, o (4096x4096), gate, up
# (11008x4096) and down (4096x11008); seed of layer l, linear j = 1000+10l+j.
STACK_LINEARS = [("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096),
                 ("o", 4096, 4096), ("gate", 11008, 4096),
                 ("up", 11008, 4096), ("down", 4096, 11008)]
STACK_LAYERS = 32
STACK_M, STACK_R, STACK_ALPHA = 4096, 16, 32.0


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def weight(N, K, seed, outlier_frac=0.0, outlier_seed=None):
    """fp32 [N, K] ~ N(0, 0.02), optionally with x10 outliers."""
    w = _rng(seed).standard_normal((N, K), dtype=np.float32) * np.float32(WEIGHT_STD)
    if outlier_frac:
        n_out = int(round(outlier_frac * N * K))
        idx = _rng(outlier_seed).choice(N * K, size=n_out, replace=False)
        flat = w.reshape(-1)
        flat[idx] *= np.float32(10.0)
    return w


def to_bf16_bits(a32):
    """fp32 -> bf16 bit patterns through torch's CPU conversion (RNE)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def normal_bf16(shape, seed, std=1.0):
    a = _rng(seed).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a = a * np.float32(std)
    return to_bf16_bits(a)


def activations(M, K, seed):
    """x [M, K] bf16 ~ N(0, 1)."""
    return normal_bf16((M, K), seed)


def adapters(N, K, r, seed_a, seed_b):
    """A [r, K], B [N, r] bf16 ~ N(0, 0.01)."""
    return (normal_bf16((r, K), seed_a, ADAPTER_STD),
            normal_bf16((N, r), seed_b, ADAPTER_STD))


def config_inputs(name, M=None):
    """All inputs of a named config: dict(w, x, A, B, dy, r, alpha, M, N, K)."""
    c = CONFIGS[name]
    N, K = c["N"], c["K"]
    M = c["M"][-1] if M is None else M
    s = c["seeds"]
    w = weight(N, K, s["w"], c.get("outliers", 0.0), s.get("outliers"))
    A, B = adapters(N, K, c["r"], s["A"], s["B"])
    return dict(w=w, x=activations(M, K, s["x"]), dy=activations(M, N, s["dy"]),
                A=A, B=B, r=c["r"], alpha=c["alpha"], M=M, N=N, K=K)


def stack_seed(layer, j):
    return 1000 + 10 * layer + j


def stack_linear_device(layer, j, M=STACK_M, device="cuda", acts=True):
    """Inputs of linear j of layer `layer` of the 7B-shaped stack, drawn on the
    device by torch's generator seeded with stack_seed(layer, j), in the order
    W, A, B, x, dY (so W alone can be drawn again from the same seed):
    W fp32 [N, K] ~ N(0, 0.02); A [r, K], B [N, r] ~ N(0, 0.01), x [M, K] and
    dY [M, N] ~ N(0, 1), all four rounded to bf16. Returns a dict of device
    tensors: x and dY are left out when acts is False, and everything but W
    when acts is None."""
    import torch
    _, N, K = STACK_LINEARS[j]
    g = torch.Generator(device=device)
    g.manual_seed(stack_seed(layer, j))
    draw = lambda shape: torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    out = {"w": draw((N, K)) * WEIGHT_STD}
    if acts is None:
        return out
    out["A"] = (draw((STACK_R, K)) * ADAPTER_STD).to(torch.bfloat16)
    out["B"] = (draw((N, STACK_R)) * ADAPTER_STD).to(torch.bfloat16)
    if acts:
        out["x"] = draw((M, K)).to(torch.bfloat16)
        out["dy"] = draw((M, N)).to(torch.bfloat16)
    return out
