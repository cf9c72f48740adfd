"""ctypes loader for libattn.so.  No fallback: a missing library is an error."""
from __future__ import annotations

import ctypes
import os
import threading

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")
_lock = threading.Lock()
_lib = None

# status codes, as in include/attn.h
ATTN_OK = 0
ATTN_E_NULL = -1
ATTN_E_SHAPE = -2
ATTN_E_HEADDIM = -3
ATTN_E_MASK = -4
ATTN_E_WORKSPACE = -5
ATTN_E_LAUNCH = -6

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_SZ = ctypes.c_size_t

SIGNATURES = {
    "attn_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P]),
    "attn_fwd_f32": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P]),
    "attn_fwd_varlen": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F,
                             _P]),
    "attn_decode_paged_workspace_size": (_SZ, [_I, _I, _I, _I, _I]),
    "attn_decode_paged": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F,
                               _P, _SZ, _P]),
    "attn_decode_paged_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                                       _I, _F, _P]),
    "attn_prefill_paged_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "attn_prefill_paged": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I,
                                _I, _F, _P, _SZ, _P]),
    "attn_bwd_workspace_size": (_SZ, [_I, _I, _I]),
    "attn_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F,
                      _P, _SZ, _P]),
    "attn_bwd_varlen": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                             _I, _I, _F, _P, _SZ, _P]),
    "attn_merge": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "attn_status_str": (ctypes.c_char_p, [_I]),
    "attn_set_fwd_sched_slots": (_I, [_I]),
}


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                raise RuntimeError(
                    f"{_LIB_PATH} is missing: build it with "
                    "`python -m exact_softmax_attention_amd.build` (there is no CPU fallback)")
            handle = ctypes.CDLL(_LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
    return _lib


def status_str(code: int) -> str:
    return lib().attn_status_str(code).decode()
