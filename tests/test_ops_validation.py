"""CPU checks of the Python wrappers' argument validation: operands whose
shapes disagree with the stored weight (or with each other) raise ValueError
from their metadata alone, before anything is handed to the library, so the
kernels never see a mismatched buffer. No GPU is touched."""
import types

import pytest
import torch

from qlora_dequant_gemm_amd import ops


def fake_weight(N, K):
    """A stand-in for a stored weight: only its shape is read before the
    shape checks fail (the real NF4Weight holds device tensors)."""
    return types.SimpleNamespace(shape=(N, K), packed=torch.empty(0, dtype=torch.uint8))


bf = lambda *s: torch.empty(s, dtype=torch.bfloat16)
N, K, M, r = 96, 128, 4, 8


@pytest.mark.parametrize("kw,msg", [
    (dict(x=bf(M, K + 64)), "x must be"),
    (dict(x=bf(K)), "two-dimensional"),
    (dict(A=bf(r, K), B=None), "both"),
    (dict(A=bf(r, K + 64), B=bf(N, r)), "A must be"),
    (dict(A=bf(r, K), B=bf(N + 1, r)), "B must be"),
    (dict(A=bf(r, K), B=bf(N, r + 1)), "B must be"),
    (dict(out=bf(M, N + 1)), "out must be"),
])
def test_forward_shape_mismatch_raises(kw, msg):
    a = dict(x=bf(M, K), A=None, B=None, out=None)
    a.update(kw)
    with pytest.raises(ValueError, match=msg):
        ops.lora_fwd(a["x"], fake_weight(N, K), a["A"], a["B"], 16.0, out=a["out"])


@pytest.mark.parametrize("kw,msg", [
    (dict(dy=bf(M, N + 8)), "dy must be"),
    (dict(A=bf(r, K), B=bf(N, r + 8)), "B must be"),
    (dict(A=bf(r + 1, K), B=bf(N, r)), "B must be"),
    (dict(out=bf(M + 1, K)), "out must be"),
])
def test_backward_shape_mismatch_raises(kw, msg):
    a = dict(dy=bf(M, N), A=None, B=None, out=None)
    a.update(kw)
    with pytest.raises(ValueError, match=msg):
        ops.bwd_dx(a["dy"], fake_weight(N, K), a["A"], a["B"], 16.0, out=a["out"])


def test_grouped_forward_shape_mismatch_raises():
    qws = [fake_weight(N, K), fake_weight(2 * N, K)]
    with pytest.raises(ValueError, match="x has K"):
        ops.lora_fwd_grouped(bf(M, K), [fake_weight(N, K), fake_weight(N, K + 64)])
    with pytest.raises(ValueError, match="one rank"):
        ops.lora_fwd_grouped(bf(M, K), qws, [bf(r, K), bf(2 * r, K)], [bf(N, r), bf(2 * N, 2 * r)])
    with pytest.raises(ValueError, match="B must be"):
        ops.lora_fwd_grouped(bf(M, K), qws, [bf(r, K), bf(r, K)], [bf(N, r), bf(N, r)])
    with pytest.raises(ValueError, match="one adapter per weight"):
        ops.lora_fwd_grouped(bf(M, K), qws, [bf(r, K)], [bf(N, r)])
    with pytest.raises(ValueError, match=r"outs\[1\]"):
        ops.lora_fwd_grouped(bf(M, K), qws, outs=[bf(M, N), bf(M, N)])


def test_adapter_grad_shape_mismatch_raises():
    x, dy = bf(M, K), bf(M, N)
    with pytest.raises(ValueError, match="dy must be"):
        ops.lora_grad(x, bf(M + 1, N), bf(r, K), bf(N, r), 16.0)
    with pytest.raises(ValueError, match="A must be"):
        ops.lora_grad(x, dy, bf(r, K + 64), bf(N, r), 16.0)
    with pytest.raises(ValueError, match="dA must be"):
        ops.lora_grad(x, dy, bf(r, K), bf(N, r), 16.0, dA=torch.empty(r, K + 1), dB=torch.empty(N, r))
    with pytest.raises(ValueError, match="dB must be"):
        ops.lora_grad(x, dy, bf(r, K), bf(N, r), 16.0, dA=torch.empty(r, K), dB=torch.empty(N, r + 1))


def test_merge_shape_mismatch_raises():
    with pytest.raises(ValueError, match="A must be"):
        ops.merge(fake_weight(N, K), bf(r, K - 64), bf(N, r), 16.0)
    with pytest.raises(ValueError, match="out must be"):
        ops.merge(fake_weight(N, K), out=bf(N, K + 64))


def test_stored_weight_sizes_checked():
    u8 = lambda n: torch.empty(n, dtype=torch.uint8)
    i8 = lambda n: torch.empty(n, dtype=torch.int8)
    f32 = lambda n: torch.empty(n, dtype=torch.float32)
    with pytest.raises(ValueError, match="packed must be"):
        ops.NF4Weight(u8(N * K // 2 - 1), i8(N * K // 64), f32(1), (N, K))
    with pytest.raises(ValueError, match="qscale must be"):
        ops.NF4Weight(u8(N * K // 2), i8(N * K // 64 + 1), f32(1), (N, K))
    with pytest.raises(ValueError, match="step must be"):
        ops.NF4Weight(u8(N * K // 2), i8(N * K // 64), f32(2), (N, K))
    with pytest.raises(ValueError, match="multiple of 64"):
        ops.NF4Weight(u8(N * 96 // 2), i8(N * 96 // 64), f32(1), (N, 96))
    with pytest.raises(ValueError, match="qscale must be"):
        ops.NF4Weight(u8(N * K // 2), torch.empty(N * K // 64, dtype=torch.uint8), f32(1), (N, K))
