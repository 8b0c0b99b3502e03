"""ctypes binding of libqlora_nf4.so (declarations mirror include/qlora_nf4.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI. Loading fails loudly when the library is missing.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("QLORA_NF4_LIB") or os.path.join(HERE, "libqlora_nf4.so")

QLORA_OK = 0
STATUS = {0: "QLORA_OK", 1: "QLORA_ERR_NULL", 2: "QLORA_ERR_SHAPE", 3: "QLORA_ERR_ALIGN",
          4: "QLORA_ERR_RANK", 5: "QLORA_ERR_WORKSPACE", 6: "QLORA_ERR_DTYPE",
          7: "QLORA_ERR_HIP", 8: "QLORA_ERR_INIT", 9: "QLORA_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 32 << 20
F32, BF16 = 0, 1

# (name, restype, argtypes) for every symbol the header declares.
_vp, _i64, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
SIGNATURES = [
    ("qlora_nf4_quantize", _i32, [_vp, _i32, _i64, _vp, _vp, _vp]),
    ("qlora_nf4_quantize_dq", _i32, [_vp, _i32, _i64, _vp, _vp, _vp, _vp, _vp]),
    ("qlora_dq_scales", _i32, [_vp, _i64, _vp, _vp, _vp]),
    ("qlora_nf4_dequant", _i32, [_vp, _vp, _vp, _i64, _vp, _vp]),
    ("qlora_workspace_bytes", _sz, [_i32, _i64, _i64, _i64, _i32]),
    ("qlora_nf4_lora_fwd", _i32, [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _i32, _f32,
                                  _vp, _vp, _sz, _vp]),
    ("qlora_set_kernel_events", _i32, [_vp, _vp]),
    ("qlora_nf4_lora_fwd_noalloc", _i32, [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _i32, _f32,
                                          _vp, _vp]),
    ("qlora_nf4_lora_fwd_grouped", _i32, [_vp, _i64, _i64, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _f32,
                                          _vp, _vp, _sz, _vp]),
    ("qlora_nf4_lora_fwd_batched", _i32, [_i32, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _f32,
                                          _vp, _vp, _sz, _vp]),
    ("qlora_workspace_bytes_batched", _sz, [_i32, _i64, _vp, _vp, _i32]),
    ("qlora_nf4_bwd_dx", _i32, [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _i32, _f32,
                                _vp, _vp, _sz, _vp]),
    ("qlora_nf4_bwd_dx_batched", _i32, [_i32, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _f32,
                                        _vp, _vp, _sz, _vp]),
    ("qlora_workspace_bytes_bwd_batched", _sz, [_i32, _i64, _vp, _vp, _i32]),
    ("qlora_q4_quantize", _i32, [_vp, _i32, _i64, _i32, _vp, _vp, _vp, _vp, _vp]),
    ("qlora_q4_dequant", _i32, [_vp, _vp, _vp, _vp, _i64, _i32, _vp, _vp]),
    ("qlora_q4_codebook", _i32, [_i32, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float)]),
    ("qlora_nf4_merge", _i32, [_vp, _vp, _vp, _i64, _i64, _vp, _vp, _i32, _f32, _vp, _vp]),
    ("qlora_lora_grad", _i32, [_vp, _vp, _i64, _i64, _i64, _vp, _vp, _i32, _f32, _vp, _vp, _i32,
                               _vp, _sz, _vp]),
    ("qlora_nf4_codebook", _i32, [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float)]),
    ("qlora_status_string", ctypes.c_char_p, [_i32]),
    ("qlora_last_hip_error", _i32, []),
    ("qlora_abi_version", _i32, []),
]

_lib = None


class QloraError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        detail = ""
        if status == 7 and _lib is not None:
            detail = f" (hipError_t {_lib.qlora_last_hip_error()})"
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}{detail}")


def lib():
    """The loaded library (loaded once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m qlora_dequant_gemm_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def check(fn, status):
    if status != QLORA_OK:
        raise QloraError(fn, status)
