"""Loads ``libmc2.so`` and declares the C ABI of ``include/mc2.h``."""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmc2.so")

# Exported entry points: name -> (restype, argtypes)
_P = C.c_void_p
_I64 = C.c_int64
_I = C.c_int
_U32 = C.c_uint32
SIGNATURES = {
    "mc2_mm_rs_local": (_I, [_P, _P, _I64, _I64, _I64, _I, _I, _I, _I, _I, _P, _P, _P, _I, _P,
                             _P, _P, _U32, _I, _P, C.c_size_t, _P]),
    "mc2_ag_mm_local": (_I, [_P, _P, _I64, _I64, _I64, _I, _I, _I, _I, _P, _P, _P, _P, _U32, _I,
                             _P, C.c_size_t, _P]),
    "mc2_ag_mm_local_inflags": (_I, [_P, _P, _I64, _I64, _I64, _I, _I, _I, _I, _P, _P, _P, _P,
                                     _U32, _I, _P, _U32, _U32, _P, _P, C.c_size_t, _P]),
    "mc2_split_workspace_size": (C.c_size_t, []),
    "mc2_set_split_policy": (_I, [_I]),
    "mc2_mm_ar_workspace_size": (C.c_size_t, [_I64, _I64, _I, _I, _I]),
    "mc2_mm_ar_local": (_I, [_P, _P, _I64, _I64, _I64, _I, _I, _I, _P, _I, _P, _P, C.c_size_t,
                             _P]),
    "mc2_ar_sum_local": (_I, [_P, _I, _I64, _I, _I, _P, _P]),
    "mc2_moe_histc": (_I, [_P, _I64, _I, _P, _P, _P]),
    "mc2_moe_permute_workspace_size": (C.c_size_t, [_I64, _I, _I]),
    "mc2_moe_permute": (_I, [_P, _I64, _I64, _P, _I, _I, _P, _P, _P, _P, _P, C.c_size_t, _P, _P]),
    "mc2_moe_permute_noalloc": (_I, [_P, _I64, _I64, _P, _I, _I, _P, _P, _P, _P, _P, _P]),
    "mc2_gmm_dispatch": (_I, [_P, _I64, _P, _P, _I, _I, _I, _I, _P, _I64, _I64, _I, _P, _I64, _P,
                              _P]),
    "mc2_gmm_combine": (_I, [_P, _I64, _P, _P, _I, _I, _I, _I, _P, _I64, _I64, _P, _I64, _P, _P]),
    "mc2_gmm_backward_workspace_size": (C.c_size_t, [_I64, _I, _I64, _I64]),
    "mc2_gmm_combine_backward": (_I, [_P, _I64, _P, _P, _I, _I, _I, _I, _P, _I64, _I64, _P, _I64,
                                      _P, _I, _P, _P, _P, C.c_size_t, _P, _P]),
    "mc2_gmm_dispatch_backward": (_I, [_P, _I64, _P, _P, _I, _I, _I, _I, _P, _I64, _I64, _P,
                                       _I64, _P, _I64, _P, _P, C.c_size_t, _P, _P]),
    "mc2_moe_unpermute": (_I, [_P, _I64, _P, _P, _I64, _I, _I64, _P, _P, _P]),
    "mc2_status_string": (C.c_char_p, [_I]),
    "mc2_version": (C.c_char_p, []),
}

_lib = None


def load() -> C.CDLL:
    """Load the built library (once). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m gemm_collective_core_amd.build`")
        lib = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib
