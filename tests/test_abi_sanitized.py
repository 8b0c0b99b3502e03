"""The C ABI layer's host code (argument checks, codebook derivation,
workspace planning, dispatch) built with AddressSanitizer and
UndefinedBehaviorSanitizer, and the CPU ABI tests run against that build in a
child process with the sanitizer runtime preloaded. Any memory error or
undefined behaviour in the host code aborts the child."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_tests_pass_under_host_sanitizers():
    if shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc not available")
    sys.path.insert(0, ROOT)
    from qlora_dequant_gemm_amd import build
    lib = build.build_sanitized()
    rt = build.sanitizer_runtime()
    if not os.path.exists(rt):
        pytest.skip("sanitizer runtime not found")
    env = dict(os.environ)
    env["LD_PRELOAD"] = rt + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["QLORA_NF4_LIB"] = lib
    probe = ("import ctypes, sys; sys.path.insert(0, %r); from qlora_dequant_gemm_amd import _lib; "
             "assert _lib.LIB_PATH == %r, _lib.LIB_PATH; _lib.lib(); "
             "assert hasattr(ctypes.CDLL(None), '__asan_init'); print('sanitized library loaded')" % (ROOT, lib))
    res = subprocess.run([sys.executable, "-c", probe], env=env, capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    res = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q",
                          "-m", "not gpu", "-p", "no:cacheprovider"],
                         env=env, capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-4000:]
    assert "passed" in res.stdout
