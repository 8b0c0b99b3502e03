#!/usr/bin/env python3
"""Benchmark of the NF4 dequant-GEMM hot path on one MI355X.

Default workload: the whole 7B-shaped frozen stack, 32 layers x {q, k, v, o
4096x4096; gate, up 11008x4096; down 4096x11008}, every linear stored as NF4
with double-quantized constants and resident in HBM (3.34 GB), LoRA r=16
(alpha 32) on all 224 linears. One step = 224 fused dequant forwards at
M = 4096 tokens in layer order, then 224 fused dequant backward dX in reverse
order; value = the step's algorithmic TFLOP/s (2MNK + 2Mr(K+N) per call).

Beside the step, in the same run:
  decode   the resident stack walked at decode shapes (M = 1, 4, 16 tokens):
           per layer the fused forward of q, k, v (one grouped call: they
           share x), o, gate and up (one grouped call), down -- every weight
           byte streamed from HBM once per walk (3.34 GB, far beyond the
           256 MB last-level cache); weight-stream GB/s per M, and the fused
           backward dX walk at M = 16.
  quantize the fp32 -> NF4 + double-quant kernel over all 224 weights, timed
           as the stack is loaded (GB/s of fp32 read + stored format written).
  context  a plain bf16 GEMM (torch.matmul on the dequantized weight) at each
           training shape, a plain streaming read of the resident stack, and
           the per-call times of every linear type.

Other workloads (--config 7b_attn, 7b_mlp_up, 65b_up, ...) time one weight:
decode configs report GB/s, training configs TFLOP/s.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFS = 2500.0     # MI355X dense bf16 MFMA, vendor figure
NF4_BYTES_PER_PARAM = 0.5 + 1 / 64 + 4 / 16384


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", default="7b_stack",
                   help="tiny, 7b_attn, 7b_mlp_up, 7b_mlp_down, 65b_up, 65b_attn or 7b_stack")
    p.add_argument("--copies", type=int, default=0, help="weight copies rotated (0 = auto)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle CPU time")
    p.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                   help="only run a plain device-to-device copy of BYTES bytes 3 times (the reference "
                        "kernel that scales the FETCH_SIZE / WRITE_SIZE counters) and exit")
    return p.parse_args()


# ---------------------------------------------------------------------------
# algorithmic work
# ---------------------------------------------------------------------------
def quantize_bytes(N, K):
    return N * K * (4 + NF4_BYTES_PER_PARAM)


def matmul_bytes(M, N, K, r, op):
    weight = N * K * NF4_BYTES_PER_PARAM
    adapters = 2 * r * (K + N)
    acts = 2 * M * K + 2 * M * N
    return weight + adapters + acts


def matmul_flops(M, N, K, r):
    return 2 * M * N * K + 2 * M * r * (K + N)


# ---------------------------------------------------------------------------
# GPU workload
# ---------------------------------------------------------------------------
class Workload:
    def __init__(self, name, copies):
        import torch
        import synth
        from qlora_dequant_gemm_amd import ops
        self.torch, self.ops = torch, ops
        c = synth.CONFIGS[name]
        self.name = name
        self.N, self.K, self.r, self.alpha = c["N"], c["K"], c["r"], c["alpha"]
        self.decode = max(c["M"]) <= 16
        self.Ms = list(c["M"])
        s = c["seeds"]
        dev = "cuda"
        N, K, r = self.N, self.K, self.r
        w = synth.weight(N, K, s["w"], c.get("outliers", 0.0), s.get("outliers"))
        w_t = torch.from_numpy(w).to(dev)
        nbytes_w = w.nbytes
        if copies <= 0:
            # enough fp32 + NF4 copies to exceed the 256 MB last-level cache twice
            copies = int(min(64, max(4, np.ceil(2 * 256e6 / (nbytes_w + N * K * NF4_BYTES_PER_PARAM)))))
            copies += copies % 2
            if max(c["M"]) <= 16:
                # decode calls read only the NF4 copy: 32 of them (>= 277 MB
                # at 4096x4096) exceed the last-level cache on their own
                copies = max(copies, 32)
        self.C = copies
        # distinct weights per copy (scaled by 1 + c/1024, same distribution shape)
        self.w = [w_t * (1.0 + i / 1024.0) for i in range(copies)]
        self.qw = [ops.quantize_weight(wi) for wi in self.w]
        bf = lambda a: torch.from_numpy(a).view(torch.bfloat16).to(dev)
        A, B = synth.adapters(N, K, r, s["A"], s["B"])
        self.A, self.B = bf(A), bf(B)
        self.x = {M: bf(synth.activations(M, K, s["x"])) for M in self.Ms}
        self.dy = {M: bf(synth.activations(M, N, s["dy"])) for M in self.Ms}
        self.bwd_M = [max(self.Ms)]
        self.y = {M: torch.empty((M, N), dtype=torch.bfloat16, device=dev) for M in self.Ms}
        self.dx = {M: torch.empty((M, K), dtype=torch.bfloat16, device=dev) for M in self.bwd_M}
        self.ws = ops.Workspace(dev)
        self.ws.get(max(ops.workspace_bytes(op, M, N, K, r) for op in (0, 1) for M in self.Ms))
        self.absmax_c = torch.empty(N * K // 64, dtype=torch.float32, device=dev)
        torch.cuda.synchronize()

    # the calls of one step, in order, as (label, fn)
    def calls(self, step):
        wl = self
        c = step % self.C
        u = (c + self.C // 2) % self.C
        out = []
        qw_dst = self.qw[c]

        def quant():
            wl.ops.quantize_dq(self.w[c], packed=qw_dst.packed, absmax=self.absmax_c, q=qw_dst.qscale,
                               step=qw_dst.step)

        out.append(("quantize_dq", quant))
        for M in self.Ms:
            out.append((f"fwd_M{M}", lambda M=M: wl.ops.lora_fwd(self.x[M], self.qw[u], self.A, self.B,
                                                                   self.alpha, out=self.y[M], ws=self.ws)))
        for M in self.bwd_M:
            out.append((f"bwd_M{M}", lambda M=M: wl.ops.bwd_dx(self.dy[M], self.qw[u], self.A, self.B,
                                                                 self.alpha, out=self.dx[M], ws=self.ws)))
        return out

    def work(self):
        """{label: (bytes, flops)} algorithmic work per call."""
        N, K, r = self.N, self.K, self.r
        wk = {"quantize_dq": (quantize_bytes(N, K), 0.0)}
        for M in self.Ms:
            wk[f"fwd_M{M}"] = (matmul_bytes(M, N, K, r, 0), matmul_flops(M, N, K, r))
        for M in self.bwd_M:
            wk[f"bwd_M{M}"] = (matmul_bytes(M, N, K, r, 1), matmul_flops(M, N, K, r))
        return wk

    def step_work(self):
        """(bytes, flops) of one step: every call once."""
        wk = self.work()
        return sum(b for b, _ in wk.values()), sum(f for _, f in wk.values())

    def timing_groups(self):
        """(label, launches) for per-call timing: one graph runs the call once per
        weight copy of the rotation, C launches back to back."""
        labels = [lab for lab, _ in self.calls(0)]
        return [(lab, [self.calls(c)[i][1] for c in range(self.C)]) for i, lab in enumerate(labels)]

    def extra_groups(self):
        """Calls timed beside the step but not part of it: decode shapes, the
        grouped forward of three weights sharing x (q, k, v of a layer); training
        shapes, the adapter gradients and the merge."""
        if self.decode:
            out = []
            N, K, r = self.N, self.K, self.r
            for M in self.Ms:
                fns = [lambda c=c, M=M: self.ops.lora_fwd_grouped(self.x[M], [self.qw[(c + i) % self.C] for i in range(3)],
                                                                  [self.A] * 3, [self.B] * 3, self.alpha, ws=self.ws)
                       for c in range(0, self.C, 3)]
                byts = 3 * (N * K * NF4_BYTES_PER_PARAM + 2 * r * (K + N) + 2 * M * N) + 2 * M * K
                out.append((f"fwd_qkv_grouped_M{M}", fns, (byts, 3 * matmul_flops(M, N, K, r))))
            self.ws.get(3 * self.ops.workspace_bytes(0, max(self.Ms), N, K, r))
            return out
        M = max(self.Ms)
        N, K, r = self.N, self.K, self.r
        dev = "cuda"
        self.dA = self.torch.empty((r, K), dtype=self.torch.float32, device=dev)
        self.dB = self.torch.empty((N, r), dtype=self.torch.float32, device=dev)
        self.ws.get(self.ops.workspace_bytes(2, M, N, K, r))
        fn = lambda: self.ops.lora_grad(self.x[M], self.dy[M], self.A, self.B, self.alpha, dA=self.dA, dB=self.dB,
                                        ws=self.ws)
        work = (2 * M * (K + N) + 4 * r * (K + N), 2 * M * r * (K + N))
        self.merged = self.torch.empty((N, K), dtype=self.torch.bfloat16, device=dev)
        qw = self.qw[self.C // 2]
        mfn = lambda: self.ops.merge(qw, self.A, self.B, self.alpha, out=self.merged)
        mwork = (N * K * (NF4_BYTES_PER_PARAM + 2) + 2 * r * (K + N), 2 * N * K * r)
        return [(f"lora_grad_M{M}", [fn] * 4, work), ("merge", [mfn] * 4, mwork)]

    def describe(self):
        shapes = {"7b_attn": "7B attention projection W 4096x4096", "7b_mlp_up": "7B MLP up W 11008x4096",
                  "7b_mlp_down": "7B MLP down W 4096x11008", "65b_up": "65B up W 22016x8192",
                  "65b_attn": "65B attention W 8192x8192", "tiny": "tiny W 256x256"}
        return (f"{shapes.get(self.name, self.name)} NF4 blk64 + int8 double-quant (blk256), "
                f"LoRA r={self.r} alpha={self.alpha:g}; step = quantize+DQ, fused fwd at "
                f"M={','.join(map(str, self.Ms))}, fused bwd dX at M={self.bwd_M[0]}")

    def config_extra(self):
        return {"N": self.N, "K": self.K, "weight_copies_rotated": self.C}


class StackWorkload:
    """The 7B-shaped frozen stack: 32 layers x {q, k, v, o 4096x4096; gate, up
    11008x4096; down 4096x11008}, every linear quantized (NF4 + double quant)
    and resident in HBM, LoRA r=16 (alpha 32) on all 224 linears. One step runs
    the 224 fused forwards at M = 4096 in layer order, then the 224 fused
    backward dX in reverse order. Each linear has its own synthetic x and dY
    (no attention, norms or activation functions between the linears); outputs
    of equal shape share a buffer. W, adapters and activations are drawn on the
    device from the per-linear seeds, W is quantized once before timing (those
    quantize launches are timed) and its fp32 copy freed."""

    name = "7b_stack"
    DECODE_M = (1, 4, 16)

    def __init__(self):
        import torch
        import synth
        from qlora_dequant_gemm_amd import ops
        self.torch, self.ops, self.synth = torch, ops, synth
        self.L, self.lin = synth.STACK_LAYERS, synth.STACK_LINEARS
        self.M, self.r, self.alpha = synth.STACK_M, synth.STACK_R, synth.STACK_ALPHA
        self.Ms, self.bwd_M, self.decode, self.C = [self.M], [self.M], False, 1
        self.lay = []
        for l in range(self.L):
            row = []
            for j in range(len(self.lin)):
                d = synth.stack_linear_device(l, j, self.M)
                d["qw"] = ops.quantize_weight(d.pop("w"))
                row.append(d)
            self.lay.append(row)
        torch.cuda.synchronize()
        # quantize + double quant, timed as the seven quantize launches of one
        # layer captured in one graph (layer 0's fp32 weights drawn again from
        # their seeds: 0.77 GB together, beyond the last-level cache), times
        # the layer count
        qin = []
        for j in range(len(self.lin)):
            w = synth.stack_linear_device(0, j, self.M, acts=None)["w"]
            N, K = w.shape
            nb = N * K // 64
            qin.append((w, torch.empty(N * K // 2, dtype=torch.uint8, device="cuda"),
                        torch.empty(nb, dtype=torch.float32, device="cuda"),
                        torch.empty(nb, dtype=torch.int8, device="cuda"),
                        torch.empty((nb + 255) // 256, dtype=torch.float32, device="cuda")))
        qstream = torch.cuda.Stream()
        g = graph_of([lambda a=a: ops.quantize_dq(a[0], packed=a[1], absmax=a[2], q=a[3], step=a[4]) for a in qin],
                     qstream)
        qms = time_graph(g, qstream, 5) * self.L
        qbytes = sum(quantize_bytes(a[0].numel(), 1) for a in qin) * self.L
        del g, qin
        self.quantize = {"ms_total": round(qms, 4), "weights": self.L * len(self.lin),
                         "GB/s": round(qbytes / qms / 1e6, 1),
                         "hbm_frac": round(qbytes / qms / 1e6 / HBM_PEAK_GBS, 4), "algorithmic_bytes": qbytes,
                         "kernel": "k_quantize",
                         "note": "fp32 W read once + NF4 codes, absmax, int8 scales and steps written once; "
                                 "the seven quantize launches of one layer (64-180 MB of fp32 each) timed as one "
                                 "graph, times the layer count"}
        self.nf4_bytes = sum(d["qw"].nbytes for row in self.lay for d in row)
        self.y = {N: torch.empty((self.M, N), dtype=torch.bfloat16, device="cuda") for _, N, _ in self.lin}
        self.dx = {K: torch.empty((self.M, K), dtype=torch.bfloat16, device="cuda") for _, _, K in self.lin}
        self.ws = ops.Workspace("cuda")
        need = max(ops.workspace_bytes(op, M, N, K, self.r) for op in (0, 1) for _, N, K in self.lin
                   for M in (self.M,) + self.DECODE_M)
        import ctypes
        from qlora_dequant_gemm_amd import _lib
        G = self.L * len(self.lin)
        Ns = (ctypes.c_int64 * G)(*[N for _ in range(self.L) for _, N, _ in self.lin])
        Ks = (ctypes.c_int64 * G)(*[K for _ in range(self.L) for _, _, K in self.lin])
        bneed = max(_lib.lib().qlora_workspace_bytes_batched(G, M, Ns, Ks, self.r) for M in self.DECODE_M)
        self.ws.get(max(need, bneed, 3 * max(ops.workspace_bytes(0, M, N, K, self.r) for _, N, K in self.lin
                                             for M in self.DECODE_M)))
        # decode inputs: one x per contraction size and M (the weights differ,
        # which is what streams), outputs per (M, N)
        g = torch.Generator(device="cuda")
        g.manual_seed(7)
        self.xd = {(M, K): torch.randn((M, K), generator=g, device="cuda").bfloat16()
                   for M in self.DECODE_M for K in (4096, 11008)}
        self.dyd = {(M, N): torch.randn((M, N), generator=g, device="cuda").bfloat16()
                    for M in self.DECODE_M for N in (4096, 11008)}
        self.yd = {(M, N): torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
                   for M in self.DECODE_M for N in (4096, 11008)}
        self.dxd = {(M, K): torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
                    for M in self.DECODE_M for K in (4096, 11008)}
        torch.cuda.synchronize()

    def _fwd(self, l, j):
        d, N = self.lay[l][j], self.lin[j][1]
        return lambda: self.ops.lora_fwd(d["x"], d["qw"], d["A"], d["B"], self.alpha, out=self.y[N], ws=self.ws)

    def _bwd(self, l, j):
        d, K = self.lay[l][j], self.lin[j][2]
        return lambda: self.ops.bwd_dx(d["dy"], d["qw"], d["A"], d["B"], self.alpha, out=self.dx[K], ws=self.ws)

    def calls(self, step):
        nl = len(self.lin)
        out = [(f"fwd_{self.lin[j][0]}", self._fwd(l, j)) for l in range(self.L) for j in range(nl)]
        out += [(f"bwd_{self.lin[j][0]}", self._bwd(l, j)) for l in reversed(range(self.L))
                for j in reversed(range(nl))]
        return out

    def timing_groups(self):
        """(label, launches): one graph runs that linear's call in all 32 layers."""
        nl = len(self.lin)
        return ([(f"fwd_{self.lin[j][0]}", [self._fwd(l, j) for l in range(self.L)]) for j in range(nl)] +
                [(f"bwd_{self.lin[j][0]}", [self._bwd(l, j) for l in range(self.L)]) for j in range(nl)])

    def calls_per_step(self, label):
        return self.L

    def work(self):
        wk = {}
        for name, N, K in self.lin:
            wk[f"fwd_{name}"] = (matmul_bytes(self.M, N, K, self.r, 0), matmul_flops(self.M, N, K, self.r))
            wk[f"bwd_{name}"] = (matmul_bytes(self.M, N, K, self.r, 1), matmul_flops(self.M, N, K, self.r))
        return wk

    def step_work(self):
        wk = self.work()
        return (self.L * sum(b for b, _ in wk.values()), self.L * sum(f for _, f in wk.values()))

    # -- decode walks over the resident stack ------------------------------
    def decode_walk(self, M):
        """The fused forwards of one decode pass at M tokens, in layer order:
        per layer q/k/v as one grouped call (shared x), o, gate/up as one
        grouped call, down."""
        ops, a, ws = self.ops, self.alpha, self.ws
        x4, x11 = self.xd[(M, 4096)], self.xd[(M, 11008)]
        fns = []
        for l in range(self.L):
            q, k, v, o, gt, up, dn = self.lay[l]
            fns.append(lambda q=q, k=k, v=v: ops.lora_fwd_grouped(
                x4, [q["qw"], k["qw"], v["qw"]], [q["A"], k["A"], v["A"]], [q["B"], k["B"], v["B"]], a, ws=ws))
            fns.append(lambda o=o: ops.lora_fwd(x4, o["qw"], o["A"], o["B"], a, out=self.yd[(M, 4096)], ws=ws))
            fns.append(lambda gt=gt, up=up: ops.lora_fwd_grouped(
                x4, [gt["qw"], up["qw"]], [gt["A"], up["A"]], [gt["B"], up["B"]], a, ws=ws))
            fns.append(lambda dn=dn: ops.lora_fwd(x11, dn["qw"], dn["A"], dn["B"], a, out=self.yd[(M, 4096)],
                                                  ws=ws))
        return fns

    def decode_batched(self, M):
        """All 224 fused forwards of one decode pass as one batched call (the
        linears of this synthetic stack do not depend on one another): one
        launch per 32 weights."""
        ops, a, ws = self.ops, self.alpha, self.ws
        ds = [d for row in self.lay for d in row]
        xs = [self.xd[(M, self.lin[j][2])] for _ in range(self.L) for j in range(len(self.lin))]
        outs = [self.yd[(M, self.lin[j][1])] for _ in range(self.L) for j in range(len(self.lin))]
        return [lambda: ops.lora_fwd_batched(xs, [d["qw"] for d in ds], [d["A"] for d in ds],
                                             [d["B"] for d in ds], a, outs=outs, ws=ws)]

    def decode_bwd_walk(self, M):
        """The fused backward dX of every linear at M tokens, layers in reverse."""
        ops, a, ws = self.ops, self.alpha, self.ws
        fns = []
        for l in reversed(range(self.L)):
            for j in reversed(range(len(self.lin))):
                _, N, K = self.lin[j]
                d = self.lay[l][j]
                fns.append(lambda d=d, N=N, K=K: ops.bwd_dx(self.dyd[(M, N)], d["qw"], d["A"], d["B"], a,
                                                            out=self.dxd[(M, K)], ws=ws))
        return fns

    def decode_bwd_batched(self, M):
        """All 224 backward dX at M tokens as one batched call (one launch
        per 32 weights; the linears of this synthetic stack do not depend on
        one another)."""
        ops, a, ws = self.ops, self.alpha, self.ws
        ds = [d for row in self.lay for d in row]
        dys = [self.dyd[(M, self.lin[j][1])] for _ in range(self.L) for j in range(len(self.lin))]
        outs = [self.dxd[(M, self.lin[j][2])] for _ in range(self.L) for j in range(len(self.lin))]
        return [lambda: ops.bwd_dx_batched(dys, [d["qw"] for d in ds], [d["A"] for d in ds],
                                           [d["B"] for d in ds], a, outs=outs, ws=ws)]

    def walk_bytes(self, M):
        """Algorithmic bytes of one walk: every weight's stored format and
        adapters once, plus each call's activations in and out."""
        return sum(matmul_bytes(M, N, K, self.r, 0) for _, N, K in self.lin) * self.L

    def describe(self):
        return (f"7B-shaped frozen stack: {self.L} layers x {{q,k,v,o 4096x4096; gate,up 11008x4096; "
                f"down 4096x11008}}, NF4 blk64 + int8 double-quant (blk256) resident in HBM "
                f"({self.nf4_bytes} B), LoRA r={self.r} alpha={self.alpha:g} on all "
                f"{self.L * len(self.lin)} linears; step = {self.L * len(self.lin)} fused fwd at M={self.M} "
                f"in layer order, then {self.L * len(self.lin)} fused bwd dX in reverse")

    def extra_groups(self):
        return []

    def config_extra(self):
        return {"layers": self.L, "linears": [list(t) for t in self.lin], "nf4_resident_bytes": self.nf4_bytes}


def graph_of(fns, stream):
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for fn in fns:
            fn()
    g.replay()
    torch.cuda.synchronize()
    return g


def time_graph(g, stream, reps):
    """ms per replay of a captured graph, from events on its stream."""
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def time_eager(fn, stream, reps):
    """ms per call of fn issued eagerly on `stream` (after two warm-up calls)."""
    import torch
    with torch.cuda.stream(stream):
        fn()
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def run_gpu(args):
    """Step time and per-call times, both from graph replays timed with events."""
    import torch
    wl = StackWorkload() if args.config == "7b_stack" else Workload(args.config, args.copies)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for s in range(args.warmup):
            for _, fn in wl.calls(s):
                fn()
    torch.cuda.synchronize()
    # one graph per weight-copy phase of the rotation; each holds one full step
    graphs = []
    for c in range(wl.C):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _, fn in wl.calls(c):
                fn()
        graphs.append(g)
    torch.cuda.synchronize()
    for s in range(args.warmup):
        graphs[s % wl.C].replay()
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        start.record(stream)
        for s in range(args.steps):
            graphs[(args.warmup + s) % wl.C].replay()
        end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / args.steps
    print(f"# step: {ms_step:.4f} ms ({args.steps} steps, {wall:.2f} s wall)", file=sys.stderr, flush=True)
    del graphs

    # per-call durations: for each call, one graph runs its launches back to
    # back (single matrix: once per weight copy of the rotation; stack: that
    # linear in every layer); events on the launch stream bracket `reps`
    # replays of that graph
    per_call = {}
    extra = {}
    groups = [(lab, fns, None) for lab, fns in wl.timing_groups()] + wl.extra_groups()
    for lab, fns, work in groups:
        reps = max(2, args.steps // len(fns))
        g = graph_of(fns, stream)
        ms = time_graph(g, stream, reps) / len(fns)
        del g
        if work is None:
            per_call[lab] = ms
        else:
            extra[lab] = {"ms": round(ms, 5), "GB/s": round(work[0] / ms / 1e6, 1),
                          "hbm_frac": round(work[0] / ms / 1e6 / HBM_PEAK_GBS, 4),
                          "TFLOP/s": round(work[1] / ms / 1e9, 2)}
    wl.extra = extra
    wl.kernel_ms = kernel_times(wl, stream, max(wl.Ms))
    wl.decode_result = decode_walks(wl, stream) if isinstance(wl, StackWorkload) else None
    return wl, ms_step, per_call, wall


def decode_walks(wl, stream, reps=10):
    """Weight-stream rate of the decode walks over the resident stack."""
    out = {}
    for M in wl.DECODE_M:
        g = graph_of(wl.decode_walk(M), stream)
        ms = time_graph(g, stream, reps)
        del g
        b = wl.walk_bytes(M)
        out[f"fwd_M{M}"] = {"ms": round(ms, 4), "GB/s": round(b / ms / 1e6, 1),
                            "hbm_frac": round(b / ms / 1e6 / HBM_PEAK_GBS, 4), "bytes": b,
                            "launch_groups": 4 * wl.L}
        print(f"# decode walk M={M}: {ms:.4f} ms, {b / ms / 1e6:.1f} GB/s", file=sys.stderr, flush=True)
        g = graph_of(wl.decode_batched(M), stream)
        ms = time_graph(g, stream, reps)
        del g
        out[f"fwd_batched_M{M}"] = {"ms": round(ms, 4), "GB/s": round(b / ms / 1e6, 1),
                                    "hbm_frac": round(b / ms / 1e6 / HBM_PEAK_GBS, 4), "bytes": b,
                                    "launches": -(-len(wl.lin) * wl.L // 32)}
        print(f"# decode batched M={M}: {ms:.4f} ms, {b / ms / 1e6:.1f} GB/s", file=sys.stderr, flush=True)
    M = 16
    g = graph_of(wl.decode_bwd_walk(M), stream)
    ms = time_graph(g, stream, reps)
    del g
    b = wl.walk_bytes(M)
    out[f"bwd_M{M}"] = {"ms": round(ms, 4), "GB/s": round(b / ms / 1e6, 1),
                        "hbm_frac": round(b / ms / 1e6 / HBM_PEAK_GBS, 4), "bytes": b,
                        "launch_groups": len(wl.lin) * wl.L}
    print(f"# decode bwd walk M={M}: {ms:.4f} ms", file=sys.stderr, flush=True)
    g = graph_of(wl.decode_bwd_batched(M), stream)
    ms = time_graph(g, stream, reps)
    del g
    out[f"bwd_batched_M{M}"] = {"ms": round(ms, 4), "GB/s": round(b / ms / 1e6, 1),
                                "hbm_frac": round(b / ms / 1e6 / HBM_PEAK_GBS, 4), "bytes": b,
                                "launches": -(-len(wl.lin) * wl.L // 32)}
    print(f"# decode bwd batched M={M}: {ms:.4f} ms, {b / ms / 1e6:.1f} GB/s", file=sys.stderr, flush=True)
    return out


def sclk_under_load(stream):
    """The shader clock the driver reports while a burst of bf16 matmuls runs
    (sysfs pp_dpm_sclk, the level marked current), or None where unreadable."""
    import glob
    import torch
    paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    if not paths:
        return None
    a = torch.randn((8192, 8192), device="cuda").bfloat16()
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    seen = []
    with torch.cuda.stream(stream):
        for _ in range(200):
            torch.matmul(a, a, out=b)
    for _ in range(5):
        time.sleep(0.02)
        for p in paths:
            try:
                for line in open(p):
                    if line.strip().endswith("*"):
                        seen.append(int(line.split(":")[1].strip().rstrip("*").strip().lower().rstrip("mhz")))
            except (OSError, ValueError, IndexError):
                pass
    torch.cuda.synchronize()
    return max(seen) if seen else None


def context_figures(wl, stream):
    """Plain ROCm-library and streaming figures beside the fused kernels:
    torch.matmul (hipBLASLt) in bf16 on the dequantized weight at each
    training shape, plain streaming read and copy rates of HBM, and the shader
    clock under load."""
    import torch
    ops = wl.ops
    out = {"bf16_gemm_on_dequantized_weight": {}}
    seen = {}
    for j, (name, N, K) in enumerate(wl.lin):
        if (N, K) in seen:
            continue
        seen[(N, K)] = name
        d = wl.lay[0][j]
        wdq = ops.dequant(d["qw"])
        x, dy = d["x"], d["dy"]
        yb = torch.empty((wl.M, N), dtype=torch.bfloat16, device="cuda")
        db = torch.empty((wl.M, K), dtype=torch.bfloat16, device="cuda")
        f = 2 * wl.M * N * K
        mf = time_eager(lambda: torch.matmul(x, wdq.t(), out=yb), stream, 10)
        mb = time_eager(lambda: torch.matmul(dy, wdq, out=db), stream, 10)
        out["bf16_gemm_on_dequantized_weight"][f"{name} {N}x{K}"] = {
            "fwd_ms": round(mf, 4), "fwd_TFLOP/s": round(f / mf / 1e9, 1),
            "bwd_ms": round(mb, 4), "bwd_TFLOP/s": round(f / mb / 1e9, 1)}
        del wdq, yb, db
    # plain streaming figures of the same HBM: one 2 GiB fp32 read (sum) and
    # one 2 GiB device-to-device copy (bytes read + written), single launches
    n = (2 << 30) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    c = torch.empty_like(a)
    tot = torch.zeros((), dtype=torch.float32, device="cuda")
    ms = time_eager(lambda: torch.sum(a, dim=0, out=tot), stream, 5)
    out["stream_read_2GiB"] = {"ms": round(ms, 4), "GB/s": round(4 * n / ms / 1e6, 1), "bytes": 4 * n,
                               "how": "torch.sum over a 2 GiB fp32 tensor"}
    ms = time_eager(lambda: c.copy_(a), stream, 5)
    out["copy_2GiB"] = {"ms": round(ms, 4), "GB/s": round(8 * n / ms / 1e6, 1), "bytes": 8 * n,
                        "how": "torch copy_ of a 2 GiB fp32 tensor, bytes read + written"}
    del a, c
    out["sclk_mhz_under_load"] = sclk_under_load(stream)
    return out


def cpu_baseline(args, wl):
    import synth
    from oracle import gemm, nf4
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    cores = len(os.sched_getaffinity(0))
    c = synth.CONFIGS[wl.name]
    s = c["seeds"]
    N, K, r, alpha = wl.N, wl.K, wl.r, wl.alpha
    # sample: slices of whole rows of W (a row slice is a smaller instance of
    # the same per-row work: quantize + DQ + dequant of those rows and the
    # matmuls against them), taken in turn until about --cpu-seconds of oracle
    # time has been spent; the rate is scaled to the step's algorithmic bytes
    w = synth.weight(N, K, s["w"], c.get("outliers", 0.0), s.get("outliers"))
    A, B = synth.adapters(N, K, r, s["A"], s["B"])
    xs = {M: synth.activations(M, K, s["x"]) for M in wl.Ms}
    dys = {M: synth.activations(M, N, s["dy"]) for M in wl.bwd_M}
    step_bytes = wl.step_work()[0]
    rows = min(N, 256)                      # multiple of 4: 1024 weights = whole DQ groups
    done_rows = 0
    t_total = 0.0
    passes = 0
    while t_total < args.cpu_seconds and t_total < 120.0:
        n0 = (passes * rows) % N
        sl = slice(n0, min(N, n0 + rows))
        ws = w[sl]
        nrow = ws.shape[0]
        t = time.perf_counter()
        packed, q, step, _ = nf4.quantize_all(ws)
        wd = nf4.dequantize(packed, q, step).reshape(nrow, K)
        for M in wl.Ms:
            gemm.lora_forward(xs[M], wd, A, B[sl], alpha, r)
        for M in wl.bwd_M:
            gemm.backward_dx(dys[M][:, sl], wd, A, B[sl], alpha, r)
        t_total += time.perf_counter() - t
        done_rows += nrow
        passes += 1
    total_bytes = step_bytes * done_rows / N
    return {"value": total_bytes / t_total / 1e9, "unit": "GB/s", "cores": int(max(1, blas_threads)),
            "host_cores": cores, "kind": "oracle",
            "sample": f"{passes} oracle passes over {rows}-row slices of W {N}x{K} ({done_rows} rows = "
                      f"{done_rows / N:.3f} of one step): quantize + double-quant + dequant (numpy, one "
                      f"thread) and the fp64 forward at M={','.join(map(str, wl.Ms))} and backward dX at "
                      f"M={wl.bwd_M[0]} ({blas_threads} BLAS threads); {t_total:.1f} s, scaled to the "
                      f"step's algorithmic bytes"}


def cpu_baseline_stack(args, wl):
    """The oracle on row slices of layer 0's q (4096x4096), gate (11008x4096)
    and down (4096x11008), taken in turn: quantize + DQ + dequant of the slice,
    then the fp64 forward and backward dX at M = 4096 against it. A slice of
    rows is a smaller instance of the same per-row work; the rate is the
    algorithmic flops done per second, the step's unit."""
    import synth
    import torch
    from oracle import gemm, nf4
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    bits = lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)
    host = []
    for j in (0, 4, 6):
        d = synth.stack_linear_device(0, j, wl.M)
        host.append(dict(w=d["w"].cpu().numpy(), A=bits(d["A"]), B=bits(d["B"]), x=bits(d["x"]),
                         dy=bits(d["dy"])))
        del d
    torch.cuda.empty_cache()
    rows, M, r, alpha = 256, wl.M, wl.r, wl.alpha
    flops = 0.0
    t_total = 0.0
    passes = 0
    while t_total < args.cpu_seconds and t_total < 120.0:
        h = host[passes % 3]
        N, K = h["w"].shape
        n0 = (passes // 3 * rows) % N
        sl = slice(n0, min(N, n0 + rows))
        nrow = sl.stop - sl.start
        t = time.perf_counter()
        packed, q, step, _ = nf4.quantize_all(h["w"][sl])
        wd = nf4.dequantize(packed, q, step).reshape(nrow, K)
        gemm.lora_forward(h["x"], wd, h["A"], h["B"][sl], alpha, r)
        gemm.backward_dx(h["dy"][:, sl], wd, h["A"], h["B"][sl], alpha, r)
        t_total += time.perf_counter() - t
        flops += 2 * matmul_flops(M, nrow, K, r)
        passes += 1
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": int(max(1, blas_threads)),
            "host_cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{passes} oracle passes over {rows}-row slices of layer 0's q, gate and down in turn: "
                      f"quantize + double-quant + dequant (numpy, one thread), fp64 forward and backward dX "
                      f"at M={M} ({blas_threads} BLAS threads); {t_total:.1f} s, {flops / 1e12:.2f} TFLOP"}


# ---------------------------------------------------------------------------
# HBM traffic of the dominant kernel, from committed counter summaries
# ---------------------------------------------------------------------------
CSRC = os.path.join(ROOT, "qlora_dequant_gemm_amd", "csrc")
# call label -> (kernel, translation unit that defines it)
CALL_KERNEL = {"quantize_dq": ("k_quantize", "quant.hip"), "fwd": ("k_dec_fwd", "decode.hip"),
               "fwd_big": ("k_gemm_fwd", "gemm.hip"), "bwd": ("k_bwd_small", "small.hip"),
               "bwd_big": ("k_gemm_bwd", "gemm.hip")}


def kernel_times(wl, stream, M, reps_max=32):
    """Per call label whose main kernel is a matmul: ms of that kernel alone,
    from HIP events the library records on the launch stream right before and
    after it (qlora_set_kernel_events), averaged over the label's calls. The
    calls are issued back to back, each with its own pair of events, so the
    stream never waits for the host between an event and its kernel."""
    import ctypes
    import torch
    from qlora_dequant_gemm_amd import _lib
    hip = ctypes.CDLL("libamdhip64.so")
    for fn in ("hipEventCreate", "hipEventSynchronize", "hipEventElapsedTime", "hipEventDestroy"):
        getattr(hip, fn).restype = ctypes.c_int
    hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    ev = [(ctypes.c_void_p(), ctypes.c_void_p()) for _ in range(reps_max)]
    made = []
    L = _lib.lib()
    out = {}
    try:
        for e0, e1 in ev:
            if hip.hipEventCreate(ctypes.byref(e0)) or hip.hipEventCreate(ctypes.byref(e1)):
                raise RuntimeError("hipEventCreate failed")
            made += [e0, e1]
        for lab, fns in wl.timing_groups():
            if kernel_of(lab, M)[0] == "k_quantize":
                continue
            with torch.cuda.stream(stream):
                fns[0]()
            torch.cuda.synchronize()
            calls = fns[:reps_max]
            with torch.cuda.stream(stream):
                for fn, (e0, e1) in zip(calls, ev):
                    L.qlora_set_kernel_events(e0, e1)
                    fn()
            L.qlora_set_kernel_events(None, None)
            tot = 0.0
            for _, (e0, e1) in zip(calls, ev):
                ms = ctypes.c_float()
                if hip.hipEventSynchronize(e1) or hip.hipEventElapsedTime(ctypes.byref(ms), e0, e1):
                    raise RuntimeError(f"kernel events of {lab} not recorded")
                tot += ms.value
            out[lab] = tot / len(calls)
    finally:
        L.qlora_set_kernel_events(None, None)
        torch.cuda.synchronize()
        for e in made:
            hip.hipEventDestroy(e)
    return out


def kernel_of(label, M):
    """(kernel, source) that does the arithmetic of a call label."""
    key = label if label == "quantize_dq" else label.split("_")[0]
    if key in ("fwd", "bwd") and M > 16:
        key += "_big"
    return CALL_KERNEL[key]


def source_digest(unit):
    """sha256 over a translation unit and every local header it includes."""
    import hashlib
    import re
    seen, todo = [], [unit]
    while todo:
        f = todo.pop()
        if f in seen:
            continue
        seen.append(f)
        text = open(os.path.join(CSRC, f)).read()
        todo += [g for g in re.findall(r'#include "([^"]+)"', text) if os.path.exists(os.path.join(CSRC, g))]
    h = hashlib.sha256()
    for f in sorted(seen):
        h.update(f.encode())
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def read_traffic(kernel, unit, config):
    """Bytes per launch from profiles/<kernel>_<config>_traffic.txt, or None when
    there is no such summary or the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{config}_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_digest") != source_digest(unit):
        return None
    return float(kv["traffic_bytes_per_launch"])


def copy_probe(nbytes):
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": a.numel() * 4}), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        sys.stderr.write("bench.py measures one GPU only: the NF4 dequant-GEMM hot path runs on a single "
                         "MI355X here; --gpus N > 1 is not supported.\n")
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        sys.stderr.write("bench.py needs a GPU\n")
        sys.exit(1)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    wl, ms_step, per_call, wall = run_gpu(args)
    wk = wl.work()
    step_bytes, step_flops = wl.step_work()
    kernels = {}
    for lab, ms in per_call.items():
        b, f = wk[lab]
        kernels[lab] = {"ms": round(ms, 5), "GB/s": round(b / ms / 1e6, 1),
                        "hbm_frac": round(b / ms / 1e6 / HBM_PEAK_GBS, 4)}
        if lab in wl.kernel_ms:
            kernels[lab]["kernel_ms"] = round(wl.kernel_ms[lab], 5)
        if f:
            kernels[lab]["TFLOP/s"] = round(f / ms / 1e9, 2)
    # the roofline kernel: the one with the largest share of the step's time
    # (its own launch time x calls per step, summed over the calls that run
    # it; per-call time where a call has no marked kernel)
    share = {}
    for lab, call_ms in per_call.items():
        ms = wl.kernel_ms.get(lab, call_ms)
        kn = kernel_of(lab, max(wl.Ms))
        n = wl.calls_per_step(lab) if hasattr(wl, "calls_per_step") else 1
        t, b_, f_, labs = share.get(kn, (0.0, 0.0, 0.0, []))
        share[kn] = (t + n * ms, b_ + n * wk[lab][0], f_ + n * wk[lab][1], labs + [lab])
    (kname, unit_src), (t_k, b_k, f_k, labs_k) = max(share.items(), key=lambda kv: kv[1][0])
    traffic = read_traffic(kname, unit_src, wl.name)
    n_launch = sum(wl.calls_per_step(l) if hasattr(wl, "calls_per_step") else 1 for l in labs_k)
    call_ms = sum((wl.calls_per_step(l) if hasattr(wl, "calls_per_step") else 1) * per_call[l] for l in labs_k)
    common = {"traffic": traffic, "kernel": kname, "calls": labs_k, "launches_per_step": n_launch,
              "ms_per_launch": round(t_k / n_launch, 5), "step_time_share": round(t_k / ms_step, 4),
              "timing": "kernel alone, between HIP events the library records around its launch on the call's "
                        "stream (qlora_set_kernel_events), averaged over the calls",
              "call_ms_per_launch": round(call_ms / n_launch, 5)}
    if wl.decode or kname == "k_quantize":
        ach = b_k / t_k / 1e6
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_launch": b_k / n_launch}
    else:
        ach = f_k / t_k / 1e9
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                "frac": round(ach / MFMA_BF16_PEAK_TFS, 4), "algorithmic_flops_per_launch": f_k / n_launch}
    roof.update(common)
    metric = "fused NF4-dequant GEMM TFLOP/s + weight-stream GB/s (% of MI355X roofline)"
    if wl.decode:
        value, unit = step_bytes / ms_step / 1e6, "GB/s"
    else:
        value, unit = step_flops / ms_step / 1e9, "TFLOP/s"
    config = {"workload": wl.describe(), "name": wl.name, "M": wl.Ms, "r": wl.r, "alpha": wl.alpha,
              "parallelism": "single GPU"}
    config.update(wl.config_extra())
    line = {
        "metric": metric, "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": config,
        "roofline": roof,
        "kernels": kernels,
        "step_bytes": step_bytes, "step_flops": step_flops,
    }
    if getattr(wl, "decode_result", None):
        dec = wl.decode_result
        fw = [v for k, v in dec.items() if k.startswith("fwd_batched")]
        tb, tm = sum(v["bytes"] for v in fw), sum(v["ms"] for v in fw)
        ach = tb / tm / 1e6
        line["decode"] = dict(dec, note="the resident stack walked at M tokens. fwd_M: per layer q/k/v (one "
                                        "grouped call), o, gate/up (one grouped call), down -- 128 dependent "
                                        "launches; fwd_batched_M: all 224 linears in one batched call (7 "
                                        "launches; the synthetic linears are independent). bytes = every "
                                        "weight's stored format + adapters + activations once; bwd_M16: the "
                                        "backward dX of all 224 linears at M = 16, one call each in reverse "
                                        "layer order (224 dependent launches); bwd_batched_M16: the same as "
                                        "one batched call (7 launches)")
        line["roofline_decode"] = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": round(ach / HBM_PEAK_GBS, 4), "kernel": "k_dec_fwd",
                                   "traffic": read_traffic("k_dec_fwd", "decode.hip", "7b_stack_decode"),
                                   "over": "batched fwd walks at M = " + ", ".join(str(m) for m in wl.DECODE_M)}
        line["quantize"] = wl.quantize
        line["context"] = context_figures(wl, torch.cuda.Stream())
    if wl.extra:
        line["outside_step"] = dict(wl.extra, note="timed alone at the step's shapes: decode, one grouped "
                                                   "forward of three weights sharing x (qlora_nf4_lora_fwd_"
                                                   "grouped); training, adapter gradients dA, dB "
                                                   "(qlora_lora_grad; GB/s counts x and dY read once and "
                                                   "dA, dB written) and the adapter merged into one bf16 "
                                                   "weight (qlora_nf4_merge; NF4 read + bf16 written)")
    if not args.no_cpu_baseline:
        if isinstance(wl, StackWorkload):
            line["cpu_baseline"] = cpu_baseline_stack(args, wl)
        else:
            line["cpu_baseline"] = cpu_baseline(args, wl)
            if unit == "TFLOP/s":
                cb = line["cpu_baseline"]
                cb["value"] = cb["value"] * step_flops / step_bytes / 1e3
                cb["unit"] = "TFLOP/s"
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
