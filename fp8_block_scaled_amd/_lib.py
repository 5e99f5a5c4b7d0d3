"""ctypes loader for libfp8bs.so and the raw C entry points (pointer-level API).

The library is built in-tree by ``fp8_block_scaled_amd.build``.  There is no
fallback: if the library is missing or fails to load, every call raises.
"""

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# FP8BS_LIBRARY names another build of the same library (the host-sanitized build
# that the ABI validation tests load); by default the in-tree libfp8bs.so.
LIB_PATH = os.environ.get("FP8BS_LIBRARY") or os.path.join(_PKG, "libfp8bs.so")

# Header constants (include/fp8bs.h).
FP8BS_OK = 0
STATUS_NAMES = {
    0: "FP8BS_OK",
    -1: "FP8BS_ERR_NULL",
    -2: "FP8BS_ERR_SHAPE",
    -3: "FP8BS_ERR_ALIGN",
    -4: "FP8BS_ERR_DEVICE",
    -5: "FP8BS_ERR_HIP",
    -6: "FP8BS_ERR_WORKSPACE",
    -7: "FP8BS_ERR_VALUE",
}

# Every symbol the header declares, with (restype, argtypes).
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
SIGNATURES = {
    "fp8_quant_act": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P]),
    "fp8_quant_weight": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P]),
    "fp8_silu_mul_quant": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _P]),
    "fp8_rmsnorm_quant": (ctypes.c_int, [_P, _P, ctypes.c_float, _P, _P, _I64, _I64, _P]),
    "fp8_block_linear": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P, ctypes.c_size_t, _P]),
    "fp8_block_linear_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _P]),
    "fp8_block_linear_workspace_size": (ctypes.c_size_t, [_I64, _I64, _I64]),
    "nvfp4_w4a16_linear": (ctypes.c_int, [_P, _P, _P, ctypes.c_float, _P, _I64, _I64, _I64, _P, ctypes.c_size_t, _P]),
    "nvfp4_w4a16_workspace_size": (ctypes.c_size_t, [_I64, _I64, _I64]),
    "fp8bs_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "fp8bs_abi_version": (ctypes.c_int, []),
}

_lib = None


class Fp8bsError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        text = lib().fp8bs_status_string(status).decode()
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(status, status)} ({text})")


def lib():
    """The loaded library (loads on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m fp8_block_scaled_amd.build` "
                "(the HIP path has no CPU fallback)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def check(fn_name, status):
    if status != FP8BS_OK:
        raise Fp8bsError(fn_name, status)
