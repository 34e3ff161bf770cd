"""ctypes view of libfa.so (the C ABI declared in include/fa.h)."""
from __future__ import annotations

import ctypes
import os
import threading

from . import build as _build

FA_F32 = 0
FA_MASK_BLOCK_Q = 128
FA_MASK_BLOCK_K = 64
FA_BF16 = 1
FA_F16 = 2
FA_MAX_SPLITS = 64
FA_NOALLOC_SCRATCH_BYTES = 68 * 1024 * 1024

STATUS = {
    0: "FA_OK", 1: "FA_ERR_NULLPTR", 2: "FA_ERR_SHAPE", 3: "FA_ERR_GQA",
    4: "FA_ERR_HEAD_DIM", 5: "FA_ERR_DTYPE", 6: "FA_ERR_WINDOW", 7: "FA_ERR_ALIGN",
    8: "FA_ERR_HIP", 9: "FA_ERR_WORKSPACE", 10: "FA_ERR_SPLITS", 11: "FA_ERR_STRIDE",
    12: "FA_ERR_MASK",
}

# Every symbol include/fa.h declares, with its ctypes signature.
_P, _I, _F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
SIGNATURES = {
    "fa_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I, _P]),
    "fa_fwd_ex": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I, _I, _P]),
    "fa_fwd_noalloc": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I, _I, _P]),
    "fa_fwd_strided": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P,
                            _F, _I, _I, _I, _I, _P]),
    "fa_fwd_block_sparse": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _I, _I,
                                 _F, _I, _I, _I, _I, _P]),
    "fa_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I,
                    _P]),
    "fa_bwd_strided": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                            _P, _P, _P, _P, _P, _P, _P, _P, _F, _I, _I, _I, _P]),
    "fa_bwd_block_sparse": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                                 _P, _I, _I, _F, _I, _I, _I, _P]),
    "fa_plan_splits": (_I, [_I, _I, _I, _I, _I, _I, _I, _I, _I]),
    "fa_bwd_plan": (_I, [_I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _P]),
    "fa_schedule_table": (_I, [_I, _I, _I, _I, _I, _I, _I, _I, _I, _I, _P, _I, _P]),
    "fa_status_string": (ctypes.c_char_p, [_I]),
    "fa_release": (None, []),
}

_lock = threading.Lock()
_lib = None


def lib() -> ctypes.CDLL:
    """Load libfa.so (building it first if it has never been built)."""
    global _lib
    with _lock:
        if _lib is None:
            path = _build.ensure_built()
            handle = ctypes.CDLL(path)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
        return _lib


def library_path() -> str:
    return _build.LIB_PATH


class FaError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        text = lib().fa_status_string(status).decode()
        super().__init__(f"{STATUS.get(status, status)}: {text}")
