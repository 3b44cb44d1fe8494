"""ctypes loader for libfox.so (the HIP kernels behind the C ABI in include/fox.h).

There is no fallback: if the library is missing or fails to load, every entry
point raises.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# FOX_LIBRARY selects another build of the same library (the host-sanitizer check build).
LIB_PATH = os.environ.get("FOX_LIBRARY") or os.path.join(_HERE, "libfox.so")

FOX_OK = 0
FOX_ERR_INVALID_ARG = 1
FOX_ERR_UNSUPPORTED = 2
FOX_ERR_WORKSPACE = 3
FOX_ERR_HIP = 4
FOX_ERR_SCRATCH = 5
FOX_DECODE_SCRATCH_BYTES = 16 << 20  # include/fox.h
FOX_F32 = 0
FOX_BF16 = 1
FOX_HEAD_MAJOR = 0
FOX_TOKEN_MAJOR = 1

# exported symbol -> (restype, argtypes)
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
SIGNATURES = {
    "fox_logf_cumsum": (ctypes.c_int, [_P, _P, _I64, _I64, _P]),
    "fox_attn_fwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, ctypes.c_float,
                                    ctypes.c_int, _P]),
    "fox_attn_fwd_ex": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, ctypes.c_float,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int, _P]),
    "fox_attn_fwd_noncausal": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, ctypes.c_float,
                                              ctypes.c_int, _P]),
    "fox_attn_fwd_pruned_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64, _I64]),
    "fox_attn_fwd_pruned": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _I64, _I64, _I64, _I64,
                                           ctypes.c_float, ctypes.c_int, _P]),
    "fox_attn_decode_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64, _I64]),
    "fox_attn_decode": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _I64, _I64, _I64, _I64,
                                       ctypes.c_float, ctypes.c_int, _P]),
    "fox_attn_decode_noalloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, ctypes.c_float,
                                               ctypes.c_int, _P]),
    "fox_attn_decode_ragged": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _I64, _I64, _I64,
                                              _I64, ctypes.c_float, ctypes.c_int, _P]),
    "fox_attn_decode_paged": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _I64, _I64,
                                             _I64, _I64, _I64, _I64, ctypes.c_float, ctypes.c_int, _P]),
    "fox_attn_bwd_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64, _I64]),
    "fox_attn_bwd": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _I64, _I64, _I64,
                                    _I64, ctypes.c_float, ctypes.c_int, ctypes.c_int, _P]),
    "fox_attn_bwd_ex": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _I64, _I64,
                                       _I64, _I64, ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int, _P]),
    "fox_attn_bwd_staged_workspace_bytes": (ctypes.c_size_t, [_I64, _I64, _I64, _I64]),
    "fox_attn_bwd_staged": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _I64, _I64,
                                           _I64, _I64, ctypes.c_float, ctypes.c_int, ctypes.c_int, _P]),
    "fox_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}

_lib = None


class FoxError(RuntimeError):
    """A libfox entry point returned a non-OK status."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: status {status} ({status_string(status)})")


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libfox.so not built at {LIB_PATH}; run python -m forget_gated_causal_amd.build")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().fox_status_string(int(status)).decode()


def check(fn: str, status: int) -> None:
    if status != FOX_OK:
        raise FoxError(fn, status)
