"""ctypes view of libspa2.so (include/spa2.h). Argument marshalling only."""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libspa2.so")

OK, E_NULL, E_SHAPE, E_DTYPE, E_PARAM, E_WORKSPACE, E_HIP, E_ALIGN, E_SCRATCH = range(9)
NOALLOC_SCRATCH_BYTES = 32 << 20  # SPA2_NOALLOC_SCRATCH_BYTES
F32, BF16 = 0, 1


class Desc(C.Structure):
    _fields_ = [("B", C.c_int32), ("H", C.c_int32), ("N", C.c_int32), ("D", C.c_int32),
                ("BQ", C.c_int32), ("BKV", C.c_int32), ("dtype", C.c_int32)]


class BlockMaskC(C.Structure):
    _fields_ = [("mask", C.c_void_p), ("row_cnt", C.c_void_p), ("row_idx", C.c_void_p),
                ("col_cnt", C.c_void_p), ("col_idx", C.c_void_p), ("row_order", C.c_void_p),
                ("col_order", C.c_void_p)]


# name -> (restype, argtypes)
_P, _D, _SZ = C.c_void_p, C.c_double, C.c_size_t
_DESC = C.POINTER(Desc)
_BM = C.POINTER(BlockMaskC)
SIGNATURES = {
    "spa2_status_str": (C.c_char_p, [C.c_int]),
    "spa2_last_error": (C.c_char_p, []),
    "spa2_num_blocks": (C.c_int32, [C.c_int32, C.c_int32]),
    "spa2_pool": (C.c_int, [_DESC, _P, _P, _P, _P, _P]),
    "spa2_mask_workspace_size": (C.c_int, [_DESC, C.POINTER(_SZ)]),
    "spa2_mask": (C.c_int, [_DESC, _P, _P, _D, _D, _BM, _P, _P, _SZ, _P]),
    "spa2_select": (C.c_int, [_DESC, _P, _D, _D, _BM, _P]),
    "spa2_mask_lists": (C.c_int, [_DESC, _BM, _P]),
    "spa2_fwd": (C.c_int, [_DESC, _P, _P, _P, _BM, _P, _P, _P, _P]),
    "spa2_bwd_workspace_size": (C.c_int, [_DESC, C.POINTER(_SZ)]),
    "spa2_bwd_workspace_bytes": (_SZ, [_DESC]),
    "spa2_bwd": (C.c_int, [_DESC, _P, _P, _P, _P, _P, _P, _P, _BM, _P, _P, _P, _P, _SZ, _P]),
    "spa2_bwd_noalloc": (C.c_int, [_DESC, _P, _P, _P, _P, _P, _P, _P, _BM, _P, _P, _P, _P]),
    "spa2_bwd_prep": (C.c_int, [_DESC, _P, _P, _P, _P, _P]),
    "spa2_bwd_dkdv": (C.c_int, [_DESC, _P, _P, _P, _P, _P, _P, _BM, _P, _P, _P]),
    "spa2_bwd_dq": (C.c_int, [_DESC, _P, _P, _P, _P, _P, _P, _SZ, _BM, _P, _P]),
    "spa2_error_terms": (C.c_int, [_DESC, _P, _P, _P, _P, _P, _P, _P]),
    "spa2_bwd_dq_rowterm": (C.c_int, [_DESC, _P, _P, _P, _P, _P, _P, _P, _BM, _P, _SZ, _P, _P]),
}

_lib = None


def lib() -> C.CDLL:
    """Load libspa2.so once. Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing; build it with "
                "`python -m block_sparse_attention_spa2_amd.build` (hipcc, gfx950)")
        handle = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


class Spa2Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        L = lib()
        msg = L.spa2_status_str(status).decode()
        detail = L.spa2_last_error().decode() if status == E_HIP else ""
        super().__init__(f"{fn} failed: status {status} ({msg}){' ' + detail if detail else ''}")
        self.status = status


def check(fn: str, status: int) -> None:
    if status != OK:
        raise Spa2Error(fn, status)
