"""ctypes declarations of libbased.so (the C ABI in include/based.h).

Loading fails loudly if the library has not been built; there is no
fallback implementation anywhere in this package.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbased.so")

BASED_OK, BASED_E_INVALID, BASED_E_UNSUPPORTED, BASED_E_LAUNCH, BASED_E_TOO_LARGE = 0, 1, 2, 3, 4
BASED_F32, BASED_BF16 = 0, 1

# Every function the header declares, with (restype, argtypes).
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_S = ctypes.c_size_t
SIGNATURES = {
    "based_num_features": (_I, [_I]),
    "based_status_string": (ctypes.c_char_p, [_I]),
    "based_prefill_workspace_bytes": (_S, [_I, _I, _I, _I, _I]),
    "based_prefill": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _I, _P, _S, _P]),
    "based_prefill_noalloc": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _I, _P]),
    "based_decode_step": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P]),
    "swa_forward": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P]),
    "swa_cache_fill": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P]),
    "swa_decode_step": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P, _P, _P]),
    "based_hybrid_prefill_workspace_bytes": (_S, [_I, _I, _I, _I, _I]),
    "based_hybrid_prefill": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _I, _F, _I, _P, _P, _P,
                                  _I, _P, _S, _P]),
    "based_prefill_backward_workspace_bytes": (_S, [_I, _I, _I, _I, _I]),
    "based_prefill_backward": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _P, _P, _S, _P]),
    "based_swa_backward_workspace_bytes": (_S, [_I, _I, _I]),
    "based_swa_backward": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P, _S, _P]),
}

_lib = None


class BasedError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib().based_status_string(status).decode()
        super().__init__(f"{fn} failed: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m linear_attention_sequence_taylor_amd.build` (needs ROCm hipcc)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def check(fn: str, status: int) -> None:
    if status != BASED_OK:
        raise BasedError(fn, status)
