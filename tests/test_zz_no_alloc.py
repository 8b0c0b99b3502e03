"""The allocation-free forward (built-in per-GPU scratch) against the forward
that takes a workspace: same kernels, same plan, so the outputs are compared
bit for bit, on two calls in a row with the second smaller than the first
(the scratch keeps the first call's contents). Covers the decode shapes,
whose split partials and arrival counters live in the scratch, and the tiled
shapes, whose LoRA down-projection goes through it.
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qops():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from qlora_dequant_gemm_amd import ops
    return ops


def _dev(a):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.cuda()


def _case(qops, M, N, K, r, seed):
    w = synth.weight(N, K, seed)
    qw = qops.quantize_weight(_dev(w))
    x = _dev(synth.activations(M, K, seed + 1))
    if r:
        A, B = synth.adapters(N, K, r, seed + 2, seed + 3)
        A, B = _dev(A), _dev(B)
    else:
        A = B = None
    return qw, x, A, B


def _bits(t):
    return t.view(torch.int16).cpu().numpy()


# (first call, second smaller call): M, N, K, r
SEQUENCES = [
    ((16, 4096, 4096, 16), (1, 1024, 1024, 16)),       # decode, K split: partials + counters
    ((16, 11008, 4096, 64), (4, 4096, 11008, 8)),      # decode, ranks past 16, ragged K/256
    ((300, 2048, 4096, 16), (40, 512, 1024, 16)),      # tiled forward, split down-projection
    ((8, 2048, 2048, 0), (2, 256, 512, 0)),            # no adapter
]


@pytest.mark.parametrize("first,second", SEQUENCES)
def test_noalloc_matches_workspace_forward(qops, first, second):
    alpha = 32.0
    for i, (M, N, K, r) in enumerate((first, second)):
        print(f"noalloc case M={M} N={N} K={K} r={r}", flush=True)
        qw, x, A, B = _case(qops, M, N, K, r, 7100 + 10 * i + M)
        ref = qops.lora_fwd(x, qw, A, B, alpha)
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        before = torch.cuda.memory_allocated()
        got = qops.lora_fwd_noalloc(x, qw, A, B, alpha, out=out)
        assert torch.cuda.memory_allocated() <= before      # no tensor allocated by the call
        assert got.data_ptr() == out.data_ptr()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(got), _bits(ref)), f"call {i}: {(M, N, K, r)}"
        # a second identical call through the same scratch: same bits
        again = qops.lora_fwd_noalloc(x, qw, A, B, alpha)
        assert np.array_equal(_bits(again), _bits(ref))


def test_noalloc_rejects_sizes_beyond_the_scratch(qops):
    from qlora_dequant_gemm_amd import _lib
    M, N, K, r = 1 << 18, 64, 64, 128               # t = x . A^T alone is 64 MiB
    need = qops.workspace_bytes(0, M, N, K, r)
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    packed = torch.zeros(N * K // 2, dtype=torch.uint8, device="cuda")
    qscale = torch.zeros(N * K // 64, dtype=torch.int8, device="cuda")
    step = torch.zeros(max(1, N * K // 64 // 256), dtype=torch.float32, device="cuda")
    A = torch.zeros((r, K), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((N, r), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    st = _lib.lib().qlora_nf4_lora_fwd_noalloc(
        x.data_ptr(), M, N, K, packed.data_ptr(), qscale.data_ptr(), step.data_ptr(), A.data_ptr(),
        B.data_ptr(), r, 32.0, y.data_ptr(), None)
    assert _lib.STATUS[st] == "QLORA_ERR_SCRATCH"
