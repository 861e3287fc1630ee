"""ctypes loader for libfa_mi355x.so (the C ABI declared in include/fa.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa_mi355x.so")

FA_OK = 0
FA_ERR_INVALID_ARG = 1
FA_ERR_UNSUPPORTED = 2
FA_ERR_WORKSPACE = 3
FA_ERR_HIP = 4
FA_BF16 = 0
FA_FP32 = 1

STATUS_NAMES = {
    FA_OK: "FA_OK",
    FA_ERR_INVALID_ARG: "FA_ERR_INVALID_ARG",
    FA_ERR_UNSUPPORTED: "FA_ERR_UNSUPPORTED",
    FA_ERR_WORKSPACE: "FA_ERR_WORKSPACE",
    FA_ERR_HIP: "FA_ERR_HIP",
}

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_SZ = ctypes.c_size_t

# name -> (restype, argtypes); must match include/fa.h.
SIGNATURES = {
    "fa_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _P]),
    "fa_fwd_window": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _I, _I, _P]),
    "fa_fwd_varlen": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I, _I, _P]),
    "fa_fwd_blocksparse": (_I, [_P, _P, _P, _P, _P, _P, ctypes.c_longlong, _I, _I, _I, _I, _I, _F, _I, _I, _P]),
    "fa_bwd_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I]),
    "fa_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _I, _I, _I, _I, _I, _F, _I, _I, _P]),
    "fa_bwd_stage": (_I, [_I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _I, _I, _I, _I, _I, _F, _I, _I, _P]),
    "fa_bwd_atomic_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I]),
    "fa_bwd_atomic": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _I, _I, _I, _I, _I, _F, _I, _I, _P]),
    "fa_bwd_atomic_stage": (_I, [_I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _I, _I, _I, _I, _I, _F, _I, _I,
                                 _P]),
    "fa_bwd_window": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _I, _I, _I, _I, _I, _F, _I, _I, _I, _I, _P]),
    "fa_decode_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "fa_decode_kvcache": (_I, [_P, _P, _P, _P, _P, _P, _P, _SZ, _I, _I, _I, _I, _I, _F, _I, _I, _I, _P]),
    "fa_decode_kvcache_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _I, _P]),
    "fa_decode_kvcache_ext": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _SZ, _I, _I, _I, _I, _I, _F,
                                   _I, _I, _I, _P]),
    "fa_last_error": (ctypes.c_char_p, []),
    "fa_version": (ctypes.c_char_p, []),
}

_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library once; raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python -m exact_attention_19_amd.build` "
            "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != FA_OK:
        raise FaError(status, load().fa_last_error().decode())
