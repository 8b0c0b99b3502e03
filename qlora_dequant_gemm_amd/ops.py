"""PyTorch-facing wrappers of the C ABI (device tensors in, device tensors out).

PyTorch supplies device memory and the current HIP stream; the arithmetic is
all in the library's kernels. bf16 tensors are passed as their 16-bit
patterns, which is what the ABI expects.
"""
import ctypes

import torch

from . import _lib

BLOCK = 64
DQ_GROUP = 256


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, dtype, name, device=None, shape=None):
    """Checks, in this order: a tensor, of `dtype`, of `shape` (when given),
    on the GPU (on `device` when given), contiguous. Shapes are checked before
    the device, so that mismatches are caught from metadata alone."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class NF4Weight:
    """Stored frozen weight [N, K]: packed codes, int8 scales, fp32 steps."""

    def __init__(self, packed, qscale, step, shape):
        self.packed, self.qscale, self.step = packed, qscale, step
        self.shape = tuple(int(d) for d in shape)
        if len(self.shape) != 2:
            raise ValueError("an NF4 weight is two-dimensional [N, K]")
        N, K = self.shape
        nb = N * K // BLOCK
        if N < 1 or K < BLOCK or K % BLOCK:
            raise ValueError(f"an NF4 weight needs N >= 1 and K a multiple of {BLOCK}, got [{N}, {K}]")
        parts = [(packed, torch.uint8, N * K // 2, "packed"), (qscale, torch.int8, nb, "qscale"),
                 (step, torch.float32, (nb + DQ_GROUP - 1) // DQ_GROUP, "step")]
        for t, dt, n, name in parts:
            _shape(t, (n,), name)
            if t.dtype != dt:
                raise ValueError(f"{name} must be {dt}, got {t.dtype}")
        for t, dt, n, name in parts:
            _need(t, dt, name, packed.device, shape=(n,))

    @property
    def nbytes(self):
        return self.packed.nbytes + self.qscale.nbytes + self.step.nbytes


def quantize(w, packed=None, absmax=None):
    """fp32 or bf16 weight -> (packed uint8, absmax fp32). Flat block order."""
    if w.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("weight must be float32 or bfloat16")
    _need(w, w.dtype, "w")
    numel = w.numel()
    if packed is None:
        packed = torch.empty(numel // 2, dtype=torch.uint8, device=w.device)
    if absmax is None:
        absmax = torch.empty(numel // BLOCK, dtype=torch.float32, device=w.device)
    _need(packed, torch.uint8, "packed")
    _need(absmax, torch.float32, "absmax")
    if packed.numel() != numel // 2 or absmax.numel() != numel // BLOCK:
        raise ValueError("output buffers have the wrong size")
    wdt = _lib.F32 if w.dtype == torch.float32 else _lib.BF16
    _lib.check("qlora_nf4_quantize", _lib.lib().qlora_nf4_quantize(
        _ptr(w), wdt, numel, _ptr(packed), _ptr(absmax), _stream(w.device)))
    return packed, absmax


def dq_scales(absmax, q=None, step=None):
    _need(absmax, torch.float32, "absmax")
    nb = absmax.numel()
    if q is None:
        q = torch.empty(nb, dtype=torch.int8, device=absmax.device)
    if step is None:
        step = torch.empty((nb + DQ_GROUP - 1) // DQ_GROUP, dtype=torch.float32, device=absmax.device)
    _need(q, torch.int8, "qscale")
    _need(step, torch.float32, "step")
    if q.numel() != nb or step.numel() != (nb + DQ_GROUP - 1) // DQ_GROUP:
        raise ValueError("output buffers have the wrong size")
    _lib.check("qlora_dq_scales", _lib.lib().qlora_dq_scales(
        _ptr(absmax), nb, _ptr(q), _ptr(step), _stream(absmax.device)))
    return q, step


def quantize_dq(w, packed=None, absmax=None, q=None, step=None):
    """Quantize + double-quantize in one kernel: (packed, absmax, qscale, step)."""
    if w.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("weight must be float32 or bfloat16")
    _need(w, w.dtype, "w")
    numel = w.numel()
    nb = numel // BLOCK
    ng = (nb + DQ_GROUP - 1) // DQ_GROUP
    dev = w.device
    packed = torch.empty(numel // 2, dtype=torch.uint8, device=dev) if packed is None else packed
    absmax = torch.empty(nb, dtype=torch.float32, device=dev) if absmax is None else absmax
    q = torch.empty(nb, dtype=torch.int8, device=dev) if q is None else q
    step = torch.empty(ng, dtype=torch.float32, device=dev) if step is None else step
    for t, dt, n, name in [(packed, torch.uint8, numel // 2, "packed"), (absmax, torch.float32, nb, "absmax"),
                           (q, torch.int8, nb, "qscale"), (step, torch.float32, ng, "step")]:
        _need(t, dt, name)
        if t.numel() != n:
            raise ValueError(f"{name} has the wrong size")
    wdt = _lib.F32 if w.dtype == torch.float32 else _lib.BF16
    _lib.check("qlora_nf4_quantize_dq", _lib.lib().qlora_nf4_quantize_dq(
        _ptr(w), wdt, numel, _ptr(packed), _ptr(absmax), _ptr(q), _ptr(step), _stream(dev)))
    return packed, absmax, q, step


def quantize_weight(w):
    """Full storage format of a 2-D weight [N, K]: NF4 codes + double-quantized constants."""
    packed, _, q, step = quantize_dq(w)
    return NF4Weight(packed, q, step, w.shape)


def dequant(qw, out=None):
    numel = qw.packed.numel() * 2
    dev = qw.packed.device
    out = _check_out(out, qw.shape, dev, "out")
    _lib.check("qlora_nf4_dequant", _lib.lib().qlora_nf4_dequant(
        _ptr(qw.packed), _ptr(qw.qscale), _ptr(qw.step), numel, _ptr(out), _stream(dev)))
    return out


def workspace_bytes(op, M, N, K, r):
    return int(_lib.lib().qlora_workspace_bytes(op, M, N, K, r))


class Workspace:
    """Grow-only device scratch buffer reused across calls on one stream.

    Zero-filled when allocated: a workspace starts with the arrival counters
    of the split-K fix-ups, which must be zero before a call and are left zero
    by every call."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf = None

    def get(self, nbytes):
        if nbytes == 0:
            return None
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=self.device)
        return self.buf


def _shape(t, shape, name):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {tuple(shape)}, got {tuple(t.shape)}")


def _rows(t, name):
    if not isinstance(t, torch.Tensor) or t.dim() != 2:
        raise ValueError(f"{name} must be a two-dimensional tensor")
    return t.shape[0]


def _adapter_rank(A, B, N, K):
    """Rank of the adapter pair A [r, K], B [N, r] (0 for none); shapes only."""
    if (A is None) != (B is None):
        raise ValueError("A and B must both be given or both be None")
    if A is None:
        return 0
    r = _rows(A, "A")
    _shape(A, (r, K), "A")
    _shape(B, (N, r), "B")
    return r


def _check_adapters(A, B, N, K, dev):
    """Rank of the adapter pair A [r, K], B [N, r] (0 for none), checked."""
    r = _adapter_rank(A, B, N, K)
    if r:
        _need(A, torch.bfloat16, "A", dev, shape=(r, K))
        _need(B, torch.bfloat16, "B", dev, shape=(N, r))
    return r


def _check_out(out, shape, dev, name):
    if out is None:
        return torch.empty(shape, dtype=torch.bfloat16, device=dev)
    _need(out, torch.bfloat16, name, dev, shape=shape)
    return out


def _check_weight(qw, dev):
    if qw.packed.device != dev:
        raise ValueError("the stored weight must be on the input's device")


def lora_fwd(x, qw, A=None, B=None, alpha=0.0, out=None, ws=None):
    """y = x . deq(W)^T + (alpha/r) . (x . A^T) . B^T, all bf16 [M, K] -> [M, N]."""
    N, K = qw.shape
    M = _rows(x, "x")
    _shape(x, (M, K), "x")
    _adapter_rank(A, B, N, K)
    if out is not None:
        _shape(out, (M, N), "out")
    _need(x, torch.bfloat16, "x")
    _check_weight(qw, x.device)
    r = _check_adapters(A, B, N, K, x.device)
    out = _check_out(out, (M, N), x.device, "out")
    need = workspace_bytes(0, M, N, K, r)
    wsb = (ws or Workspace(x.device)).get(need)
    _lib.check("qlora_nf4_lora_fwd", _lib.lib().qlora_nf4_lora_fwd(
        _ptr(x), M, N, K, _ptr(qw.packed), _ptr(qw.qscale), _ptr(qw.step), _ptr(A), _ptr(B), r,
        float(alpha), _ptr(out), _ptr(wsb), 0 if wsb is None else wsb.numel(), _stream(x.device)))
    return out


def lora_fwd_noalloc(x, qw, A=None, B=None, alpha=0.0, out=None):
    """lora_fwd without a workspace: the library's built-in per-GPU scratch
    holds the split partials (nothing is allocated when `out` is given)."""
    N, K = qw.shape
    M = _rows(x, "x")
    _shape(x, (M, K), "x")
    _adapter_rank(A, B, N, K)
    if out is not None:
        _shape(out, (M, N), "out")
    _need(x, torch.bfloat16, "x")
    _check_weight(qw, x.device)
    r = _check_adapters(A, B, N, K, x.device)
    out = _check_out(out, (M, N), x.device, "out")
    _lib.check("qlora_nf4_lora_fwd_noalloc", _lib.lib().qlora_nf4_lora_fwd_noalloc(
        _ptr(x), M, N, K, _ptr(qw.packed), _ptr(qw.qscale), _ptr(qw.step), _ptr(A), _ptr(B), r,
        float(alpha), _ptr(out), _stream(x.device)))
    return out


def lora_fwd_grouped(x, qws, As=None, Bs=None, alpha=0.0, outs=None, ws=None):
    """The forward of several weights sharing x (one launch for M <= 16):
    returns [x . deq(W_i)^T + (alpha/r) . (x . A_i^T) . B_i^T for each i]."""
    M = _rows(x, "x")
    K = x.shape[1]
    G = len(qws)
    if (As is None) != (Bs is None) or (As is not None and (len(As) != G or len(Bs) != G)):
        raise ValueError("As and Bs must both be None or both hold one adapter per weight")
    if outs is not None and len(outs) != G:
        raise ValueError("one output per weight")
    Ns = [qw.shape[0] for qw in qws]
    ranks = set()
    for i, qw in enumerate(qws):
        if qw.shape[1] != K:
            raise ValueError(f"weight {i} is {qw.shape}, x has K = {K}")
        ranks.add(_adapter_rank(As[i] if As is not None else None, Bs[i] if Bs is not None else None, Ns[i], K))
        if outs is not None:
            _shape(outs[i], (M, Ns[i]), f"outs[{i}]")
    if len(ranks) != 1:
        raise ValueError("every weight of a group must have adapters of one rank")
    r = ranks.pop()
    _need(x, torch.bfloat16, "x")
    for i, qw in enumerate(qws):
        _check_weight(qw, x.device)
        _check_adapters(As[i] if As is not None else None, Bs[i] if Bs is not None else None, Ns[i], K, x.device)
    if outs is None:
        outs = [torch.empty((M, n), dtype=torch.bfloat16, device=x.device) for n in Ns]
    outs = [_check_out(o, (M, n), x.device, f"outs[{i}]") for i, (o, n) in enumerate(zip(outs, Ns))]
    arr = lambda ts: (ctypes.c_void_p * G)(*[t.data_ptr() if t is not None else 0 for t in ts])
    need = G * workspace_bytes(0, M, max(Ns), K, r)
    wsb = (ws or Workspace(x.device)).get(need)
    _lib.check("qlora_nf4_lora_fwd_grouped", _lib.lib().qlora_nf4_lora_fwd_grouped(
        _ptr(x), M, K, G, arr([q.packed for q in qws]), arr([q.qscale for q in qws]), arr([q.step for q in qws]),
        (ctypes.c_int64 * G)(*Ns), arr(As) if r else None, arr(Bs) if r else None, r, float(alpha), arr(outs),
        _ptr(wsb), 0 if wsb is None else wsb.numel(), _stream(x.device)))
    return outs


def lora_fwd_batched(xs, qws, As=None, Bs=None, alpha=0.0, outs=None, ws=None):
    """The forward of independent linears, each with its own input:
    [x_i . deq(W_i)^T + (alpha/r) . (x_i . A_i^T) . B_i^T for each i], every x_i
    [M, K_i] with one M. Decode shapes stream all weights in one launch per
    32 of them."""
    G = len(qws)
    if len(xs) != G:
        raise ValueError("one input per weight")
    if (As is None) != (Bs is None) or (As is not None and (len(As) != G or len(Bs) != G)):
        raise ValueError("As and Bs must both be None or both hold one adapter per weight")
    if outs is not None and len(outs) != G:
        raise ValueError("one output per weight")
    M = _rows(xs[0], "xs[0]")
    ranks = set()
    for i, (x, qw) in enumerate(zip(xs, qws)):
        N, K = qw.shape
        _shape(x, (M, K), f"xs[{i}]")
        ranks.add(_adapter_rank(As[i] if As is not None else None, Bs[i] if Bs is not None else None, N, K))
        if outs is not None:
            _shape(outs[i], (M, N), f"outs[{i}]")
    if len(ranks) != 1:
        raise ValueError("every weight must have adapters of one rank")
    r = ranks.pop()
    dev = xs[0].device
    for i, (x, qw) in enumerate(zip(xs, qws)):
        _need(x, torch.bfloat16, f"xs[{i}]", dev)
        _check_weight(qw, dev)
        _check_adapters(As[i] if As is not None else None, Bs[i] if Bs is not None else None, qw.shape[0],
                        qw.shape[1], dev)
    if outs is None:
        outs = [torch.empty((M, qw.shape[0]), dtype=torch.bfloat16, device=dev) for qw in qws]
    outs = [_check_out(o, (M, qw.shape[0]), dev, f"outs[{i}]") for i, (o, qw) in enumerate(zip(outs, qws))]
    arr = lambda ts: (ctypes.c_void_p * G)(*[t.data_ptr() if t is not None else 0 for t in ts])
    Ns = (ctypes.c_int64 * G)(*[qw.shape[0] for qw in qws])
    Ks = (ctypes.c_int64 * G)(*[qw.shape[1] for qw in qws])
    need = int(_lib.lib().qlora_workspace_bytes_batched(G, M, Ns, Ks, r))
    wsb = (ws or Workspace(dev)).get(need)
    _lib.check("qlora_nf4_lora_fwd_batched", _lib.lib().qlora_nf4_lora_fwd_batched(
        G, M, arr(xs), Ns, Ks, arr([q.packed for q in qws]), arr([q.qscale for q in qws]),
        arr([q.step for q in qws]), arr(As) if r else None, arr(Bs) if r else None, r, float(alpha), arr(outs),
        _ptr(wsb), 0 if wsb is None else wsb.numel(), _stream(dev)))
    return outs


def bwd_dx(dy, qw, A=None, B=None, alpha=0.0, out=None, ws=None):
    """dX = dY . deq(W) + (alpha/r) . (dY . B) . A, bf16 [M, N] -> [M, K]."""
    N, K = qw.shape
    M = _rows(dy, "dy")
    _shape(dy, (M, N), "dy")
    _adapter_rank(A, B, N, K)
    if out is not None:
        _shape(out, (M, K), "out")
    _need(dy, torch.bfloat16, "dy")
    _check_weight(qw, dy.device)
    r = _check_adapters(A, B, N, K, dy.device)
    out = _check_out(out, (M, K), dy.device, "out")
    need = workspace_bytes(1, M, N, K, r)
    wsb = (ws or Workspace(dy.device)).get(need)
    _lib.check("qlora_nf4_bwd_dx", _lib.lib().qlora_nf4_bwd_dx(
        _ptr(dy), M, N, K, _ptr(qw.packed), _ptr(qw.qscale), _ptr(qw.step), _ptr(A), _ptr(B), r,
        float(alpha), _ptr(out), _ptr(wsb), 0 if wsb is None else wsb.numel(), _stream(dy.device)))
    return out


def bwd_dx_batched(dys, qws, As=None, Bs=None, alpha=0.0, outs=None, ws=None):
    """The backward dX of independent linears, each with its own dY_i [M, N_i]:
    [dY_i . deq(W_i) + (alpha/r) . (dY_i . B_i) . A_i for each i]. Decode
    shapes stream all weights in one launch per 32 of them."""
    G = len(qws)
    if len(dys) != G:
        raise ValueError("one dy per weight")
    if (As is None) != (Bs is None) or (As is not None and (len(As) != G or len(Bs) != G)):
        raise ValueError("As and Bs must both be None or both hold one adapter per weight")
    if outs is not None and len(outs) != G:
        raise ValueError("one output per weight")
    M = _rows(dys[0], "dys[0]")
    ranks = set()
    for i, (dy, qw) in enumerate(zip(dys, qws)):
        N, K = qw.shape
        _shape(dy, (M, N), f"dys[{i}]")
        ranks.add(_adapter_rank(As[i] if As is not None else None, Bs[i] if Bs is not None else None, N, K))
        if outs is not None:
            _shape(outs[i], (M, K), f"outs[{i}]")
    if len(ranks) != 1:
        raise ValueError("every weight must have adapters of one rank")
    r = ranks.pop()
    dev = dys[0].device
    for i, (dy, qw) in enumerate(zip(dys, qws)):
        _need(dy, torch.bfloat16, f"dys[{i}]", dev)
        _check_weight(qw, dev)
        _check_adapters(As[i] if As is not None else None, Bs[i] if Bs is not None else None, qw.shape[0],
                        qw.shape[1], dev)
    if outs is None:
        outs = [torch.empty((M, qw.shape[1]), dtype=torch.bfloat16, device=dev) for qw in qws]
    outs = [_check_out(o, (M, qw.shape[1]), dev, f"outs[{i}]") for i, (o, qw) in enumerate(zip(outs, qws))]
    arr = lambda ts: (ctypes.c_void_p * G)(*[t.data_ptr() if t is not None else 0 for t in ts])
    Ns = (ctypes.c_int64 * G)(*[qw.shape[0] for qw in qws])
    Ks = (ctypes.c_int64 * G)(*[qw.shape[1] for qw in qws])
    need = int(_lib.lib().qlora_workspace_bytes_bwd_batched(G, M, Ns, Ks, r))
    wsb = (ws or Workspace(dev)).get(need)
    _lib.check("qlora_nf4_bwd_dx_batched", _lib.lib().qlora_nf4_bwd_dx_batched(
        G, M, arr(dys), Ns, Ks, arr([q.packed for q in qws]), arr([q.qscale for q in qws]),
        arr([q.step for q in qws]), arr(As) if r else None, arr(Bs) if r else None, r, float(alpha), arr(outs),
        _ptr(wsb), 0 if wsb is None else wsb.numel(), _stream(dev)))
    return outs


def lora_grad(x, dy, A, B, alpha, dA=None, dB=None, accumulate=False, ws=None):
    """Adapter gradients (dA [r, K], dB [N, r], fp32) of one QLoRA linear:
    dB = (alpha/r) . dY^T . bf16(x . A^T), dA = (alpha/r) . bf16(dY . B)^T . x.
    With accumulate=True they are added to dA and dB."""
    M = _rows(x, "x")
    _rows(dy, "dy")
    K, N = x.shape[1], dy.shape[1]
    r = _adapter_rank(A, B, N, K)
    _shape(dy, (M, N), "dy")
    if dA is not None:
        _shape(dA, (r, K), "dA")
    if dB is not None:
        _shape(dB, (N, r), "dB")
    _need(x, torch.bfloat16, "x")
    _need(dy, torch.bfloat16, "dy", x.device, shape=(M, N))
    _need(A, torch.bfloat16, "A", x.device, shape=(r, K))
    _need(B, torch.bfloat16, "B", x.device, shape=(N, r))
    if dA is None:
        dA = (torch.zeros if accumulate else torch.empty)((r, K), dtype=torch.float32, device=x.device)
    if dB is None:
        dB = (torch.zeros if accumulate else torch.empty)((N, r), dtype=torch.float32, device=x.device)
    _need(dA, torch.float32, "dA", x.device, shape=(r, K))
    _need(dB, torch.float32, "dB", x.device, shape=(N, r))
    need = workspace_bytes(2, M, N, K, r)
    wsb = (ws or Workspace(x.device)).get(need)
    _lib.check("qlora_lora_grad", _lib.lib().qlora_lora_grad(
        _ptr(x), _ptr(dy), M, N, K, _ptr(A), _ptr(B), r, float(alpha), _ptr(dA), _ptr(dB),
        1 if accumulate else 0, _ptr(wsb), 0 if wsb is None else wsb.numel(), _stream(x.device)))
    return dA, dB


NF4, INT4, FP4 = 0, 1, 2


def q4_quantize(w, fmt, double_quant=True):
    """Block-64 quantization in another 16-level format (NF4, INT4 or FP4):
    (packed, absmax, qscale, step), qscale/step None without double quantization."""
    if w.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("weight must be float32 or bfloat16")
    _need(w, w.dtype, "w")
    numel = w.numel()
    nb = numel // BLOCK
    dev = w.device
    packed = torch.empty(numel // 2, dtype=torch.uint8, device=dev)
    absmax = torch.empty(nb, dtype=torch.float32, device=dev)
    q = torch.empty(nb, dtype=torch.int8, device=dev) if double_quant else None
    step = torch.empty((nb + DQ_GROUP - 1) // DQ_GROUP, dtype=torch.float32, device=dev) if double_quant else None
    wdt = _lib.F32 if w.dtype == torch.float32 else _lib.BF16
    _lib.check("qlora_q4_quantize", _lib.lib().qlora_q4_quantize(
        _ptr(w), wdt, numel, int(fmt), _ptr(packed), _ptr(absmax), _ptr(q), _ptr(step), _stream(dev)))
    return packed, absmax, q, step


def q4_dequant(packed, fmt, absmax=None, qscale=None, step=None, out=None):
    """bf16 [numel] from a block-64 format; double-quantized constants when
    qscale/step are given, else the fp32 absmax."""
    numel = packed.numel() * 2
    dev = packed.device
    if out is None:
        out = torch.empty(numel, dtype=torch.bfloat16, device=dev)
    _need(out, torch.bfloat16, "out")
    _lib.check("qlora_q4_dequant", _lib.lib().qlora_q4_dequant(
        _ptr(packed), _ptr(absmax), _ptr(qscale), _ptr(step), numel, int(fmt), _ptr(out), _stream(dev)))
    return out


def q4_codebook(fmt):
    L = (ctypes.c_float * 16)()
    T = (ctypes.c_float * 15)()
    _lib.check("qlora_q4_codebook", _lib.lib().qlora_q4_codebook(int(fmt), L, T))
    return list(L), list(T)


def merge(qw, A=None, B=None, alpha=0.0, out=None):
    """bf16 [N, K] = bf16(deq(W) + (alpha/r) . B . A): the adapter folded into one
    dense weight (exactly the dequantized weight when there is no adapter)."""
    N, K = qw.shape
    dev = qw.packed.device
    _adapter_rank(A, B, N, K)
    if out is not None:
        _shape(out, (N, K), "out")
    r = _check_adapters(A, B, N, K, dev)
    out = _check_out(out, (N, K), dev, "out")
    _lib.check("qlora_nf4_merge", _lib.lib().qlora_nf4_merge(
        _ptr(qw.packed), _ptr(qw.qscale), _ptr(qw.step), N, K, _ptr(A), _ptr(B), r, float(alpha), _ptr(out),
        _stream(dev)))
    return out


def codebook():
    """(levels[16], thresholds[15]) as the kernels use them, host floats."""
    L = (ctypes.c_float * 16)()
    T = (ctypes.c_float * 15)()
    _lib.check("qlora_nf4_codebook", _lib.lib().qlora_nf4_codebook(L, T))
    return list(L), list(T)
