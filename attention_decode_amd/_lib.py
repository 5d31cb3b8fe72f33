"""ctypes view of libtq.so (the C ABI declared in include/tq.h).

Only argument marshalling lives here.  The library is loaded from this package
directory (or from the path in LIBTQ_PATH, e.g. an instrumented build of the
same sources); a missing library is an error, never a fallback.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("LIBTQ_PATH") or os.path.join(PKG, "libtq.so")

TQ_OK, TQ_EINVAL, TQ_EUNSUPPORTED, TQ_EALIGN, TQ_ENOMEM, TQ_EHIP, TQ_ENOTCONV = range(7)
STATUS_NAMES = ["TQ_OK", "TQ_EINVAL", "TQ_EUNSUPPORTED", "TQ_EALIGN", "TQ_ENOMEM", "TQ_EHIP",
                "TQ_ENOTCONV"]
TQ_ROT_DENSE, TQ_ROT_HADAMARD, TQ_ROT_HADAMARD2 = 0, 1, 2
TQ_F32, TQ_BF16, TQ_F16 = 0, 1, 2


class KeyFmt(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int), ("mse_bits", ctypes.c_int), ("qjl_m", ctypes.c_int),
                ("cb", ctypes.c_void_p), ("rot", ctypes.c_void_p)]


class ValFmt(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int), ("bits", ctypes.c_int), ("group", ctypes.c_int)]


class KCache(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("signs", ctypes.c_void_p),
                ("knorm", ctypes.c_void_p), ("rnorm", ctypes.c_void_p)]


class VCache(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("params", ctypes.c_void_p)]


class BlockFmt(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int), ("bits", ctypes.c_int), ("rot", ctypes.c_void_p)]


class BCache(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class CacheLayout(ctypes.Structure):
    _fields_ = [("capacity", ctypes.c_int64), ("seq_lens", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("block_size", ctypes.c_int), ("max_blocks", ctypes.c_int), ("num_blocks", ctypes.c_int64)]


# name -> (restype, argtypes); every entry point of include/tq.h
_c = ctypes
_vp, _i, _i64, _u64, _sz = _c.c_void_p, _c.c_int, _c.c_int64, _c.c_uint64, _c.c_size_t
_dp = _c.POINTER(_c.c_double)
SIGNATURES = {
    "tq_build_codebook": (_i, [_i, _i, _c.POINTER(_vp)]),
    "tq_codebook_free": (None, [_vp]),
    "tq_codebook_tables": (_i, [_vp, _dp, _dp]),
    "tq_codebook_host": (_i, [_i, _i, _dp, _dp]),
    "tq_make_rotation": (_i, [_u64, _i, _i, _c.POINTER(_vp)]),
    "tq_rotation_free": (None, [_vp]),
    "tq_rotation_host": (_i, [_u64, _i, _i, _dp, _dp]),
    "tq_key_plane_bytes": (_sz, [_c.POINTER(KeyFmt), _i64, _i]),
    "tq_val_plane_bytes": (_sz, [_c.POINTER(ValFmt), _i64, _i]),
    "tq_compress_keys": (_i, [_c.POINTER(KeyFmt), _vp, _i, _i, _i, _i64, _i64, _i64, _i64, KCache, _vp]),
    "tq_compress_values": (_i, [_c.POINTER(ValFmt), _vp, _i, _i, _i, _i64, _i64, _i64, _i64, VCache, _vp]),
    "tq_scores_workspace_bytes": (_sz, [_c.POINTER(KeyFmt), _i, _i]),
    "tq_scores": (_i, [_c.POINTER(KeyFmt), _vp, _i, _i, _i, _i, _i64, KCache, _vp, _vp, _sz, _vp]),
    "tq_attend_splits": (_i, [_c.POINTER(KeyFmt), _i, _i, _i, _i64]),
    "tq_attend_workspace_bytes": (_sz, [_c.POINTER(KeyFmt), _i, _i, _i, _i64, _i]),
    "tq_attend_decode": (_i, [_c.POINTER(KeyFmt), _c.POINTER(ValFmt), _vp, _i, _i, _i, _i, _i64,
                              KCache, VCache, _c.c_float, _i, _vp, _sz, _vp, _vp]),
    "tq_attend_decode_noalloc": (_i, [_c.POINTER(KeyFmt), _c.POINTER(ValFmt), _vp, _i, _i, _i, _i, _i64,
                                      KCache, VCache, _c.c_float, _i, _vp, _vp]),
    "tq_dequantize_keys": (_i, [_c.POINTER(KeyFmt), _i, _i, _i64, KCache, _vp, _vp]),
    "tq_append_keys": (_i, [_c.POINTER(KeyFmt), _vp, _i, _i, _i, _i, _i64, _i64, _i64, _c.POINTER(CacheLayout),
                            _vp, KCache, _vp]),
    "tq_append_values": (_i, [_c.POINTER(ValFmt), _vp, _i, _i, _i, _i, _i64, _i64, _i64, _c.POINTER(CacheLayout),
                              _vp, VCache, _vp]),
    "tq_attend_paged_workspace_bytes": (_sz, [_c.POINTER(KeyFmt), _i, _i, _i, _c.POINTER(CacheLayout), _i]),
    "tq_attend_decode_paged": (_i, [_c.POINTER(KeyFmt), _c.POINTER(ValFmt), _vp, _i, _i, _i, _i,
                                    _c.POINTER(CacheLayout), KCache, VCache, _c.c_float, _i, _vp, _sz, _vp, _vp]),
    "tq_block_plane_bytes": (_sz, [_c.POINTER(BlockFmt), _i64, _i]),
    "tq_compress_keys_block": (_i, [_c.POINTER(BlockFmt), _vp, _i, _i, _i, _i64, _i64, _i64, _i64, BCache, _vp]),
    "tq_attend_block_workspace_bytes": (_sz, [_c.POINTER(BlockFmt), _i, _i, _i, _i64, _i]),
    "tq_attend_decode_block": (_i, [_c.POINTER(BlockFmt), _c.POINTER(ValFmt), _vp, _i, _i, _i, _i, _i64, BCache,
                                    VCache, _c.c_float, _i, _vp, _sz, _vp, _vp]),
    "tq_last_error": (_c.c_char_p, []),
    "tq_profile_enable": (_i, [_i]),
    "tq_profile_read": (_i, [_c.c_char_p, _dp, _c.POINTER(_i64)]),
}

_lib = None


class TQError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__(f"{where}: {name}: {msg}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libtq.so from the package directory (build it with
    `python -m attention_decode_amd.build`)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libtq.so is not built ({LIB_PATH}); run python -m attention_decode_amd.build")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def check(status: int, where: str) -> None:
    if status != TQ_OK:
        raise TQError(status, where, lib().tq_last_error().decode(errors="replace"))
