"""ctypes loader of libmoe.so (the gfx950 HIP kernels behind the C ABI in include/moe.h)."""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
BF16, FP8, MXFP8, MXFP4 = 0, 1, 2, 3

# Every symbol the header declares, with (restype, argtypes).
_P, _I, _I64, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [_I]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_version": (ctypes.c_char_p, []),
    "moe_route": (_I, [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P]),
    "moe_route_mx": (_I, [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P]),
    "moe_align_capacity": (_I64, [_I, _I, _I, _I]),
    "moe_align": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P]),
    "moe_route_align": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P,
                             _P, _P]),
    "moe_preshuffle_bytes": (_I64, [_I, _I, _I, _I, _I]),
    "moe_preshuffle": (_I, [_I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_stage1_amax_floats": (_I64, [_I, _I, _I, _I, _I, _I, _I]),
    "moe_stage1": (_I, [_I, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P]),
    "moe_stage2_workspace_bytes": (_I64, [_I, _I, _I, _I, _I, _I, _I]),
    "moe_stage2": (_I, [_I, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P,
                        _SZ, _P]),
    "moe_stage2_noalloc": (_I, [_I, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                                _P, _P]),
    "moe_backward_preshuffle_bytes": (_I64, [_I, _I, _I, _I]),
    "moe_backward_preshuffle": (_I, [_I, _I, _I, _P, _P, _P, _P, _P, _P]),
    "moe_backward_workspace_bytes": (_I64, [_I, _I, _I, _I, _I, _I]),
    "moe_stage1_save_preact": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P]),
    "moe_backward": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I,
                          _I, _I, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
}


class MoEError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library. Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m mixture_experts_routed_top_amd.build`"
                " (the MoE layer has no other implementation)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def check(status: int) -> None:
    if status != OK:
        L = lib()
        raise MoEError(status, f"{L.moe_status_string(status).decode()}: "
                               f"{L.moe_last_error().decode()}")
