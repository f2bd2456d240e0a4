"""ctypes view of libmxstore.so (declared in include/mxstore.h).

Loading fails loudly when the library has not been built: there is no CPU
or PyTorch fallback for any entry point.
"""

from __future__ import annotations

import ctypes
import os
import threading

from .build import LIB_PATH

MX_OK = 0
MX_E_NULL = -1
MX_E_SHAPE = -2
MX_E_STRIDE = -3
MX_E_ALIGN = -4
MX_E_RANGE = -5
MX_E_ARG = -6
MX_E_LAUNCH = -7
NOALLOC_SCRATCH_BYTES = 32 << 20  # MX_NOALLOC_SCRATCH_BYTES

# Every symbol include/mxstore.h declares.
EXPORTED = (
    "mx_row_bytes",
    "mxfp4_store",
    "mxfp4_inverse_bytes",
    "mxfp4_slot_order_advised",
    "mxfp4_build_inverse",
    "mxfp4_store_by_slot",
    "mxfp4_store_slot_order_noalloc",
    "mxfp4_gather_dequant",
    "mxfp8_rope_store",
    "nvfp4_rope_store",
    "v4_rope_store",
    "save_ring_rows",
    "fused_save_compress_norm_cr1",
    "sparse_mla_attention",
    "sparse_mla_attention_split",
    "sparse_mla_attention_workspace_bytes",
    "sparse_mla_attention_splits_advised",
    "mx_last_error",
)

_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_vp = ctypes.c_void_p

_lib = None
_lock = threading.Lock()


class MxError(ValueError):
    """A libmxstore entry point rejected its arguments (status < 0)."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"libmxstore.so is not built ({LIB_PATH}); run "
                "`python -m mxfp4_paged_cache_store_amd.build` (needs hipcc)")
        L = ctypes.CDLL(LIB_PATH)
        L.mx_row_bytes.restype = _i64
        L.mx_row_bytes.argtypes = [_i64, _i32]
        L.mxfp4_store.restype = ctypes.c_int
        L.mxfp4_store.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _i64, _i64, _i64, _i32, _vp]
        L.mxfp4_inverse_bytes.restype = _i64
        L.mxfp4_inverse_bytes.argtypes = [_i64, _i64]
        L.mxfp4_slot_order_advised.restype = ctypes.c_int
        L.mxfp4_slot_order_advised.argtypes = [_i64, _i64, _i64, _i64]
        L.mxfp4_build_inverse.restype = ctypes.c_int
        L.mxfp4_build_inverse.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _vp]
        L.mxfp4_store_by_slot.restype = ctypes.c_int
        L.mxfp4_store_by_slot.argtypes = [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i32, _vp]
        L.mxfp4_store_slot_order_noalloc.restype = ctypes.c_int
        L.mxfp4_store_slot_order_noalloc.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _i64, _i64, _i64,
                                                     _i32, _vp]
        L.mxfp4_gather_dequant.restype = ctypes.c_int
        L.mxfp4_gather_dequant.argtypes = [_vp, _i64, _i64, _i64, _i64, _i32, _vp, _i64, _vp, _i64, _vp]
        for name in ("mxfp8_rope_store", "nvfp4_rope_store", "v4_rope_store"):
            fn = getattr(L, name)
            fn.restype = ctypes.c_int
            fn.argtypes = [_vp, _vp, _vp, _i64, _i64, _vp, _i64, _i64, _i64, _vp, _i64, _i32, _i32, _vp]
        L.save_ring_rows.restype = ctypes.c_int
        L.save_ring_rows.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _i64, _i64, _i64, _i64, _vp]
        L.fused_save_compress_norm_cr1.restype = ctypes.c_int
        L.fused_save_compress_norm_cr1.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, ctypes.c_float,
                                                   _vp, _i64, _vp]
        L.sparse_mla_attention.restype = ctypes.c_int
        L.sparse_mla_attention.argtypes = [_vp, _i64, _i64, _i64, _i64, _i64, _vp, _i64, _i64, _i64,
                                           _vp, _i64, _i64, ctypes.c_float, _vp, _vp, _i64, _i64, _vp]
        L.sparse_mla_attention_split.restype = ctypes.c_int
        L.sparse_mla_attention_split.argtypes = [_vp, _i64, _i64, _i64, _i64, _i64, _vp, _i64, _i64, _i64,
                                                 _vp, _i64, _i64, ctypes.c_float, _vp, _vp, _i64, _i64,
                                                 _i32, _vp, _i64, _vp]
        L.sparse_mla_attention_workspace_bytes.restype = _i64
        L.sparse_mla_attention_workspace_bytes.argtypes = [_i64, _i64, _i64]
        L.sparse_mla_attention_splits_advised.restype = _i32
        L.sparse_mla_attention_splits_advised.argtypes = [_i64, _i64, _i64]
        L.mx_last_error.restype = ctypes.c_char_p
        L.mx_last_error.argtypes = []
        _lib = L
        return L


def check(status: int) -> None:
    if status != MX_OK:
        msg = lib().mx_last_error().decode(errors="replace")
        raise MxError(status, msg)
