"""CPU checks of the C-ABI library: it loads, exports every symbol the header
declares, derives the same codebook as the oracle bit for bit, sizes its
workspace consistently, and rejects bad arguments with status codes before
launching anything (no GPU is touched by these calls)."""
import ctypes
import os
import re

import numpy as np
import pytest

from qlora_dequant_gemm_amd import _lib, ops
from oracle import nf4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qlora_nf4.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qlora_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 10
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(n for n, _, _ in _lib.SIGNATURES) == names


def test_abi_version_and_status_strings():
    L = _lib.lib()
    assert L.qlora_abi_version() == 1
    for code in range(10):
        assert L.qlora_status_string(code)
    assert L.qlora_status_string(99) == b"unknown status"


def test_kernel_events_setting():
    L = _lib.lib()
    assert L.qlora_set_kernel_events(FAKE, V(0)) == 1
    assert L.qlora_set_kernel_events(V(0), FAKE) == 1
    assert L.qlora_set_kernel_events(V(0), V(0)) == 0


def test_codebook_bitwise_equals_oracle():
    levels, thresholds = ops.codebook()
    L = np.array(levels, np.float32)
    assert np.array_equal(L.view(np.uint32), nf4.codebook().view(np.uint32))
    # thresholds: largest fp32 not above each exact midpoint
    mids = nf4.level_midpoints()
    T = np.array(thresholds, np.float32)
    assert np.all(T.astype(np.float64) <= mids)
    assert np.all(np.nextafter(T, np.float32(2)).astype(np.float64) > mids)


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_format_codebooks_bitwise_equal_oracle(fmt):
    from oracle import formats
    levels, thresholds = ops.q4_codebook(fmt)
    L = np.array(levels, np.float32)
    assert np.array_equal(L.view(np.uint32), formats.levels(fmt).view(np.uint32))
    mids = nf4.level_midpoints(formats.levels(fmt))
    T = np.array(thresholds, np.float32)
    assert np.all(T.astype(np.float64) <= mids)
    assert np.all(np.nextafter(T, np.float32(2)).astype(np.float64) > mids)


def test_format_calls_reject_bad_arguments():
    L = _lib.lib()
    a = (ctypes.c_float * 16)()
    b = (ctypes.c_float * 15)()
    assert L.qlora_q4_codebook(3, a, b) == 6 and L.qlora_q4_codebook(-1, a, b) == 6
    assert L.qlora_q4_quantize(FAKE, 0, 64, 3, FAKE, FAKE, V(0), V(0), V(0)) == 6
    assert L.qlora_q4_quantize(FAKE, 0, 64, 1, FAKE, FAKE, FAKE, V(0), V(0)) == 1
    assert L.qlora_q4_quantize(FAKE, 0, 96, 1, FAKE, FAKE, V(0), V(0), V(0)) == 2
    assert L.qlora_q4_quantize(ODD, 0, 64, 1, FAKE, FAKE, V(0), V(0), V(0)) == 3
    assert L.qlora_q4_dequant(FAKE, V(0), V(0), V(0), 64, 1, FAKE, V(0)) == 1
    assert L.qlora_q4_dequant(FAKE, V(0), FAKE, V(0), 64, 1, FAKE, V(0)) == 1
    assert L.qlora_q4_dequant(FAKE, FAKE, V(0), V(0), 64, 5, FAKE, V(0)) == 6
    assert L.qlora_q4_dequant(FAKE, FAKE, V(0), V(0), 65, 2, FAKE, V(0)) == 2


def test_workspace_sizes():
    ws = ops.workspace_bytes
    C = 16384                                                     # arrival counters open every workspace
    assert ws(0, 4096, 11008, 4096, 0) == 0
    # bf16 t (rank padded to 32) + fp32 partials of 4 contraction splits (16 ranks)
    assert ws(0, 4096, 11008, 4096, 16) == C + 4096 * 32 * 2 + 4 * 4096 * 16 * 4
    # decode shapes: 16 row blocks of 256 x 8 splits of K (two 256-deep steps
    # each at M = 16) of fp32 partials [M][256]; one split needs nothing
    assert ws(0, 16, 4096, 4096, 16) == C + 16 * 8 * 16 * 256 * 4
    assert ws(0, 1, 4096, 4096, 16) == C + 16 * 8 * 1 * 256 * 4
    assert ws(0, 16, 8, 64, 8) == 0
    # decode-shaped backward, one weight: 64 block columns x 8 splits of the
    # rows (512 rows each), fp32 partials [64][M rounded up to 4]
    assert ws(1, 16, 4096, 4096, 0) == C + 64 * 8 * 64 * 16 * 4
    assert ws(1, 1, 4096, 4096, 16) == C + 64 * 8 * 64 * 4 * 4
    assert ws(1, 16, 512, 4096, 16) == 0                          # one split: no partials
    assert ws(1, 4096, 4096, 11008, 0) == 0
    assert ws(2, 16, 16, 64, 0) == 0 and ws(0, 0, 16, 64, 0) == 0
    for op in (0, 1, 2):
        assert ws(op, 16, 8, 64, 8) % 256 == 0
    # adapter gradients: transposed B, t^T and u^T (rank padded to 32, rows to
    # 64), and the fp32 partials of the dY and x contractions
    assert ws(3, 16, 16, 64, 8) == 0 and ws(2, 16, 16, 64, 129) == 0
    g = ws(2, 4096, 11008, 4096, 16)
    fixed = C + 16 * 11008 * 2 + 2 * 32 * 4096 * 2
    assert g >= fixed + 11008 * 16 * 4 + 4096 * 16 * 4
    assert g <= fixed + 64 * (11008 + 4096) * 16 * 4 + 5 * 256
    # the batched forward: one launch per 32 weights reuses one region
    N = (ctypes.c_int64 * 3)(4096, 11008, 4096)
    K = (ctypes.c_int64 * 3)(4096, 4096, 11008)
    b = _lib.lib().qlora_workspace_bytes_batched(3, 16, N, K, 16)
    assert b >= C and (b - C) % (16 * 256 * 4) == 0
    # training shapes: one launch per 8 weights, each with its own slice of
    # the largest single-weight size
    assert _lib.lib().qlora_workspace_bytes_batched(3, 4096, N, K, 16) == 3 * max(ws(0, 4096, n, k, 16)
                                                                                   for n, k in zip(N, K))
    N12 = (ctypes.c_int64 * 12)(*([4096] * 12))
    K12 = (ctypes.c_int64 * 12)(*([4096] * 12))
    assert _lib.lib().qlora_workspace_bytes_batched(12, 4096, N12, K12, 16) == 8 * ws(0, 4096, 4096, 4096, 16)
    assert _lib.lib().qlora_workspace_bytes_batched(0, 16, N, K, 16) == 0
    # the batched backward: one launch per 32 weights at decode shapes (one
    # region of split partials), one call after another on larger M
    assert _lib.lib().qlora_workspace_bytes_bwd_batched(3, 4096, N, K, 16) == max(ws(1, 4096, n, k, 16)
                                                                                  for n, k in zip(N, K))
    b = _lib.lib().qlora_workspace_bytes_bwd_batched(3, 16, N, K, 16)
    assert b == 0 or (b >= C and (b - C) % (64 * 16 * 4) == 0)
    N1 = (ctypes.c_int64 * 1)(4096)
    K1 = (ctypes.c_int64 * 1)(4096)
    assert _lib.lib().qlora_workspace_bytes_bwd_batched(1, 16, N1, K1, 16) == ws(1, 16, 4096, 4096, 16)
    # eight 4096 x 4096 weights take 256-column items: 16 column ranges x 4
    # splits (1024 rows each) per weight, partials [256][16]
    N8 = (ctypes.c_int64 * 8)(*([4096] * 8))
    assert _lib.lib().qlora_workspace_bytes_bwd_batched(8, 16, N8, N8, 16) == C + 8 * 16 * 4 * 256 * 16 * 4
    N1b = (ctypes.c_int64 * 1)(12)
    assert _lib.lib().qlora_workspace_bytes_bwd_batched(1, 16, N1b, K1, 16) == 0      # N not a multiple of 8
    assert _lib.lib().qlora_workspace_bytes_bwd_batched(0, 16, N, K, 16) == 0


V = ctypes.c_void_p
FAKE = V(0x10000)          # a 16-byte aligned non-null address that is never dereferenced
ODD = V(0x10008)           # not 16-byte aligned


def _fwd(x=FAKE, M=16, N=64, K=64, packed=FAKE, q=FAKE, step=FAKE, A=V(0), B=V(0), r=0, alpha=0.0,
         y=FAKE, ws=V(0), wsb=0):
    return _lib.lib().qlora_nf4_lora_fwd(x, M, N, K, packed, q, step, A, B, r, alpha, y, ws, wsb, V(0))


def _bwd(dy=FAKE, M=16, N=64, K=64, packed=FAKE, q=FAKE, step=FAKE, A=V(0), B=V(0), r=0, alpha=0.0,
         dx=FAKE, ws=V(0), wsb=None):
    if wsb is None:
        wsb = ops.workspace_bytes(1, M, N, K, r)
        ws = FAKE if wsb else V(0)
    return _lib.lib().qlora_nf4_bwd_dx(dy, M, N, K, packed, q, step, A, B, r, alpha, dx, ws, wsb, V(0))


@pytest.mark.parametrize("kwargs,status", [
    (dict(x=V(0)), 1), (dict(y=V(0)), 1), (dict(packed=V(0)), 1), (dict(q=V(0)), 1),
    (dict(step=V(0)), 1),
    (dict(M=0), 2), (dict(N=0), 2), (dict(K=0), 2), (dict(K=96), 2), (dict(K=32), 2),
    (dict(x=ODD), 3), (dict(y=ODD), 3), (dict(packed=ODD), 3),
    (dict(r=8), 1), (dict(r=8, A=FAKE), 1), (dict(A=FAKE), 4), (dict(r=-1), 4),
    (dict(r=129, A=FAKE, B=FAKE), 4),
    (dict(r=8, A=ODD, B=FAKE, ws=FAKE, wsb=1 << 20), 3),
    # K = 1024 at M = 16: the decode kernel splits K, so a workspace is needed
    (dict(r=8, A=FAKE, B=FAKE, K=1024), 5), (dict(r=8, A=FAKE, B=FAKE, ws=FAKE, wsb=16, K=1024), 5),
    (dict(r=8, A=FAKE, B=FAKE, ws=ODD, wsb=1 << 20, K=1024), 3),
    (dict(M=300, r=8, A=FAKE, B=FAKE), 5),
])
def test_forward_rejects_bad_arguments(kwargs, status):
    assert _fwd(**kwargs) == status


def _fwd_noalloc(x=FAKE, M=16, N=64, K=64, packed=FAKE, q=FAKE, step=FAKE, A=V(0), B=V(0), r=0, alpha=0.0,
                 y=FAKE):
    return _lib.lib().qlora_nf4_lora_fwd_noalloc(x, M, N, K, packed, q, step, A, B, r, alpha, y, V(0))


@pytest.mark.parametrize("kwargs,status", [
    (dict(x=V(0)), 1), (dict(y=V(0)), 1), (dict(packed=V(0)), 1), (dict(step=V(0)), 1),
    (dict(M=0), 2), (dict(K=96), 2), (dict(N=1 << 22), 2),
    (dict(x=ODD), 3), (dict(y=ODD), 3),
    (dict(r=8), 1), (dict(A=FAKE), 4), (dict(r=129, A=FAKE, B=FAKE), 4),
    # a decode shape whose split partials need more than the built-in scratch,
    # and a tiled one whose t = x . A^T does
    (dict(M=16, N=4096, K=1 << 20), 9),
    (dict(M=1 << 18, N=64, K=64, r=128, A=FAKE, B=FAKE), 9),
])
def test_noalloc_forward_rejects_before_any_launch(kwargs, status):
    """Every rejection of the allocation-free forward happens on the host,
    before the scratch is looked up or anything is launched."""
    M, N, K = kwargs.get("M", 16), kwargs.get("N", 64), kwargs.get("K", 64)
    if status == 9:
        assert ops.workspace_bytes(0, M, N, K, kwargs.get("r", 0)) > _lib.NOALLOC_SCRATCH_BYTES
    assert _fwd_noalloc(**kwargs) == status


@pytest.mark.parametrize("kwargs,status", [
    (dict(dy=V(0)), 1), (dict(dx=V(0)), 1), (dict(N=12), 2), (dict(N=0), 2), (dict(K=100), 2),
    (dict(dy=ODD), 3), (dict(dx=ODD), 3), (dict(r=4, A=FAKE), 1),
    # 4096 rows at M = 16: the decode-shaped backward splits the rows, so a
    # workspace is needed
    (dict(N=4096, ws=V(0), wsb=0), 5),
])
def test_backward_rejects_bad_arguments(kwargs, status):
    assert _bwd(**kwargs) == status


def _grad(x=FAKE, dy=FAKE, M=16, N=64, K=64, A=FAKE, B=FAKE, r=8, alpha=16.0, dA=FAKE, dB=FAKE, acc=0,
          ws=None, wsb=None):
    if wsb is None:
        wsb = ops.workspace_bytes(2, M, N, K, r)
        ws = FAKE if wsb else V(0)
    return _lib.lib().qlora_lora_grad(x, dy, M, N, K, A, B, r, alpha, dA, dB, acc, ws, wsb, V(0))


@pytest.mark.parametrize("kwargs,status", [
    (dict(x=V(0)), 1), (dict(dy=V(0)), 1), (dict(dA=V(0)), 1), (dict(dB=V(0)), 1),
    (dict(A=V(0)), 1), (dict(B=V(0)), 1),
    (dict(M=0), 2), (dict(N=12), 2), (dict(K=100), 2), (dict(acc=2), 2),
    (dict(r=0), 4), (dict(r=129), 4),
    (dict(x=ODD), 3), (dict(dy=ODD), 3), (dict(dA=ODD), 3), (dict(dB=ODD), 3), (dict(A=ODD), 3),
    (dict(ws=V(0), wsb=0), 5), (dict(ws=FAKE, wsb=256), 5), (dict(ws=ODD, wsb=1 << 30), 3),
])
def test_adapter_grad_rejects_bad_arguments(kwargs, status):
    assert _grad(**kwargs) == status


@pytest.mark.parametrize("args,status", [
    ((V(0), FAKE, FAKE, 16, 64, V(0), V(0), 0, 0.0, FAKE), 1),
    ((FAKE, FAKE, FAKE, 16, 64, V(0), V(0), 0, 0.0, V(0)), 1),
    ((FAKE, FAKE, FAKE, 0, 64, V(0), V(0), 0, 0.0, FAKE), 2),
    ((FAKE, FAKE, FAKE, 16, 96, V(0), V(0), 0, 0.0, FAKE), 2),
    ((FAKE, FAKE, FAKE, 16, 64, V(0), V(0), 0, 0.0, ODD), 3),
    ((FAKE, FAKE, FAKE, 16, 64, FAKE, V(0), 4, 1.0, FAKE), 1),
    ((FAKE, FAKE, FAKE, 16, 64, FAKE, FAKE, 129, 1.0, FAKE), 4),
    ((FAKE, FAKE, FAKE, 16, 64, ODD, FAKE, 4, 1.0, FAKE), 3),
])
def test_merge_rejects_bad_arguments(args, status):
    assert _lib.lib().qlora_nf4_merge(*args, V(0)) == status


def test_grouped_forward_rejects_bad_arguments():
    L = _lib.lib()
    P = lambda *v: (ctypes.c_void_p * len(v))(*v)
    N = lambda *v: (ctypes.c_int64 * len(v))(*v)
    f, o = 0x10000, 0x10008
    ok = dict(x=FAKE, M=4, K=64, G=2, pk=P(f, f), q=P(f, f), st=P(f, f), n=N(64, 32), A=None, B=None, r=0,
              y=P(f, f), ws=V(0), wsb=0)

    def call(**kw):
        a = dict(ok, **kw)
        return L.qlora_nf4_lora_fwd_grouped(a["x"], a["M"], a["K"], a["G"], a["pk"], a["q"], a["st"], a["n"],
                                            a["A"], a["B"], a["r"], 0.0, a["y"], a["ws"], a["wsb"], V(0))
    assert call(G=0) == 2 and call(G=9) == 2 and call(K=96) == 2 and call(n=N(64, 0)) == 2
    assert call(x=V(0)) == 1 and call(pk=P(f, 0)) == 1 and call(y=P(f, 0)) == 1 and call(r=8) == 1
    assert call(y=P(f, o)) == 3 and call(pk=P(o, f)) == 3 and call(r=129, A=P(f, f), B=P(f, f)) == 4
    assert call(r=8, A=P(f, f), B=P(f, f), K=1024) == 5    # workspace needed for the split of K


def test_quantize_dq_dequant_reject_bad_arguments():
    L = _lib.lib()
    assert L.qlora_nf4_quantize(V(0), 0, 64, FAKE, FAKE, V(0)) == 1
    assert L.qlora_nf4_quantize(FAKE, 0, 65, FAKE, FAKE, V(0)) == 2
    assert L.qlora_nf4_quantize(FAKE, 0, 0, FAKE, FAKE, V(0)) == 2
    assert L.qlora_nf4_quantize(FAKE, 5, 64, FAKE, FAKE, V(0)) == 6
    assert L.qlora_nf4_quantize(ODD, 0, 64, FAKE, FAKE, V(0)) == 3
    assert L.qlora_dq_scales(FAKE, 0, FAKE, FAKE, V(0)) == 2
    assert L.qlora_dq_scales(V(0), 4, FAKE, FAKE, V(0)) == 1
    assert L.qlora_nf4_dequant(FAKE, FAKE, FAKE, 100, FAKE, V(0)) == 2
    assert L.qlora_nf4_dequant(FAKE, FAKE, FAKE, 64, ODD, V(0)) == 3
    assert L.qlora_nf4_dequant(FAKE, V(0), FAKE, 64, FAKE, V(0)) == 1
    a = (ctypes.c_float * 16)()
    assert L.qlora_nf4_codebook(a, None) == 1


def test_thresholds_sit_well_inside_quantize_cells():
    """The quantize kernel looks codes up in 129 cells of width 1/64 (cell =
    floor(64 v + 64.5)) and re-derives a code exactly only within 1e-6 of the
    cell's threshold; that is exact if every threshold is far from a cell edge
    and no two share a cell."""
    _, thresholds = ops.codebook()
    pos = np.array(thresholds, np.float64) * 64 + 64.5
    frac = pos - np.floor(pos)
    assert np.min(np.minimum(frac, 1 - frac)) / 64 > 1e-4
    assert len(set(np.floor(pos).astype(int))) == 15


def _bwd_batched(G=2, M=16, N=(64, 64), K=(64, 64), dy=FAKE, packed=FAKE, q=FAKE, step=FAKE, A=None, B=None,
                 r=0, dx=FAKE, ws=V(0), wsb=0):
    arr = lambda v: (ctypes.c_void_p * G)(*([v] * G)) if v is not None else None
    Ns = (ctypes.c_int64 * G)(*N)
    Ks = (ctypes.c_int64 * G)(*K)
    return _lib.lib().qlora_nf4_bwd_dx_batched(G, M, arr(dy), Ns, Ks, arr(packed), arr(q), arr(step), arr(A),
                                               arr(B), r, 1.0, arr(dx), ws, wsb, V(0))


@pytest.mark.parametrize("kwargs,status", [
    (dict(dy=V(0)), 1), (dict(dx=V(0)), 1), (dict(packed=V(0)), 1),
    (dict(N=(64, 12)), 2), (dict(K=(64, 100)), 2), (dict(M=0), 2), (dict(G=0, N=(), K=()), 2),
    (dict(dy=ODD), 3), (dict(dx=ODD), 3),
    (dict(r=4), 1), (dict(r=4, A=FAKE), 1), (dict(r=129, A=FAKE, B=FAKE), 4),
    (dict(N=(4096, 64), ws=V(0), wsb=0), 5),      # the decode shape splits the 4096 rows
])
def test_batched_backward_rejects_bad_arguments(kwargs, status):
    assert _bwd_batched(**kwargs) == status


def test_size_limits_return_shape_errors():
    """Sizes the kernels' 32-bit buffer descriptors or tile numbering cannot
    address are rejected before anything is launched (N, K <= 2^21; the 256 x
    256 tile count below 2^31)."""
    big = 1 << 21
    assert _fwd(N=big + 64, K=64) == 2 and _fwd(K=big + 64) == 2
    assert _fwd(M=(1 << 31) + 1) == 2
    assert _fwd(M=1 << 31, N=big, K=64) == 2                    # 2^23 x 2^13 tiles
    assert _bwd(N=big + 8, K=64, wsb=0, ws=V(0)) == 2 and _bwd(K=big + 64, wsb=0, ws=V(0)) == 2
    assert _lib.lib().qlora_nf4_merge(FAKE, FAKE, FAKE, big + 1, 64, V(0), V(0), 0, 0.0, FAKE, V(0)) == 2
    assert _lib.lib().qlora_dq_scales(FAKE, 1 << 31, FAKE, FAKE, V(0)) == 2
    # the largest accepted sizes pass the shape checks (and stop at the
    # workspace check, so nothing is launched)
    assert _fwd(M=1 << 20, N=big, K=big, r=8, A=FAKE, B=FAKE) == 5
    assert _grad(M=512, N=big, K=64, ws=V(0), wsb=0) == 5
