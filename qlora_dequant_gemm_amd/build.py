"""Build libqlora_nf4.so for gfx950 with hipcc (run on any machine with ROCm;
no GPU is needed to compile).

    python -m qlora_dequant_gemm_amd.build
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libqlora_nf4.so")
ARCH = "gfx950"

SOURCES = ["codebook.cpp", "api.cpp", "quant.hip", "lora.hip", "small.hip", "gemm.hip", "grad.hip", "merge.hip"]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
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


def build(verbose=False, extra=()):
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + FLAGS + list(extra) + ["-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libqlora_nf4.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
