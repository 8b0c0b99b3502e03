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


# Host-side sanitizer build of the C ABI layer (argument checks, codebook
# derivation, dispatch): api.cpp and codebook.cpp with AddressSanitizer and
# UndefinedBehaviorSanitizer on their host code only, linked with the regular
# kernel objects into a separate library for the CPU ABI tests (run with the
# sanitizer runtime preloaded; nothing here is used by the product path).
SAN_SOURCES = ["codebook.cpp", "api.cpp"]
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
SAN_LIB = os.path.join(OBJ, "san", "libqlora_nf4_san.so")


def build_sanitized(verbose=False):
    if not all(os.path.exists(os.path.join(OBJ, os.path.splitext(s)[0] + ".o")) for s in SOURCES):
        build(verbose)
    san = os.path.dirname(SAN_LIB)
    os.makedirs(san, exist_ok=True)
    objs = []
    for s in SOURCES:
        if s in SAN_SOURCES:
            obj = os.path.join(san, os.path.splitext(s)[0] + ".o")
            if _run([hipcc()] + FLAGS + SAN_FLAGS + ["-c", os.path.join(CSRC, s), "-o", obj], verbose):
                raise RuntimeError("hipcc failed building the sanitizer objects")
        else:
            obj = os.path.join(OBJ, os.path.splitext(s)[0] + ".o")
        objs.append(obj)
    link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libsan"] + SAN_FLAGS + ["-o", SAN_LIB] + objs
    if _run(link, verbose):
        raise RuntimeError("hipcc failed linking the sanitizer library")
    return SAN_LIB


def sanitizer_runtime():
    """The AddressSanitizer runtime the sanitizer library expects preloaded."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    clang = os.path.join(rocm, "llvm", "bin", "clang")
    res = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return res.stdout.strip()


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized(verbose=True))
    else:
        print(build(verbose=True))
