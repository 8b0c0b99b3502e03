"""Build libqlora_nf4.so for gfx950 with hipcc (run on any machine with ROCm;
no GPU is needed to compile).

    python -m qlora_dequant_gemm_amd.build

Each translation unit is compiled to an object in parallel, then the objects
are linked into the shared library.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqlora_nf4.so")
OBJ = os.path.join(HERE, "_build")
ARCH = "gfx950"

SOURCES = ["codebook.cpp", "api.cpp", "quant.hip", "lora.hip", "small.hip", "decode.hip", "gemm.hip", "grad.hip", "merge.hip",
           "noalloc.hip"]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # Bit-exact quantize/dequant: no contraction of multiply-add into FMA, and
    # HIP's default correctly rounded fp32 division is kept.
    "-ffp-contract=off",
    # Keep the compiler from emitting packed fp32 VALU operations.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
    return res.returncode


def build(verbose=False, extra=()):
    os.makedirs(OBJ, exist_ok=True)
    jobs = []
    for s in SOURCES:
        obj = os.path.join(OBJ, os.path.splitext(s)[0] + ".o")
        jobs.append(([hipcc()] + FLAGS + list(extra) + ["-c", os.path.join(CSRC, s), "-o", obj], obj))
    workers = min(len(jobs), max(1, min(8, os.cpu_count() or 1)))
    with ThreadPoolExecutor(workers) as ex:
        rcs = list(ex.map(lambda j: _run(j[0], verbose), jobs))
    if any(rcs):
        raise RuntimeError("hipcc failed building libqlora_nf4.so")
    tmp = LIB + ".tmp"
    link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [o for _, o in jobs]
    if _run(link, verbose):
        raise RuntimeError("hipcc failed linking libqlora_nf4.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
