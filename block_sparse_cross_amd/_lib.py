"""ctypes view of libbsx's C ABI (``include/bsx.h``).

Argument marshalling only: every computation happens inside libbsx.  Loading
fails loudly when the library cannot be built or opened; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading
from ctypes import POINTER, c_char_p, c_double, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libbsx.so")

BSX_OK, BSX_E_INVALID, BSX_E_UNSUPPORTED, BSX_E_WORKSPACE, BSX_E_DEVICE = range(5)
BSX_F32, BSX_BF16 = 0, 1


class BsxError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class BsxShape(ctypes.Structure):
    _fields_ = [
        ("n_blocks", c_int32),
        ("block_size", c_int32),
        ("n_q_heads", c_int32),
        ("n_kv_heads", c_int32),
        ("head_dim", c_int32),
        ("dtype", c_int32),
        ("ctx_len", c_int64),
        ("scale", c_float),
    ]


class BsxChunks(ctypes.Structure):
    _fields_ = [
        ("n_chunks", c_int32),
        ("n_slots", c_int32),
        ("start", POINTER(c_int64)),
        ("len", POINTER(c_int64)),
        ("slot", POINTER(c_int32)),
    ]


# (name, restype, argtypes) for every function bsx.h declares
_SIGNATURES = [
    ("bsx_abi_version", c_int, []),
    ("bsx_last_error", c_char_p, []),
    ("bsx_status_string", c_char_p, [c_int]),
    ("bsx_mask_from_anchors", c_int, [POINTER(BsxShape), POINTER(c_int64), POINTER(c_int64),
                                      POINTER(c_int64), POINTER(c_int64)]),
    ("bsx_validate_mask", c_int, [POINTER(BsxShape), POINTER(c_int64), POINTER(c_int64)]),
    ("bsx_cost_workspace", c_size_t, [c_int32]),
    ("bsx_cost", c_int, [POINTER(BsxShape), c_void_p, c_void_p, POINTER(BsxChunks), c_void_p,
                         c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    ("bsx_lpt", c_int, [c_int32, POINTER(c_int64), c_int32, POINTER(c_int32), POINTER(c_int64),
                        POINTER(c_int64), POINTER(c_double)]),
    ("bsx_place", c_int, [c_int32, c_int32, POINTER(c_int64), c_int32, POINTER(c_int32),
                          POINTER(c_int64), POINTER(c_int64), POINTER(c_double)]),
    ("bsx_fwd_workspace", c_size_t, [POINTER(BsxShape), POINTER(BsxChunks)]),
    ("bsx_attn_fwd", c_int, [POINTER(BsxShape), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                             c_void_p, c_void_p, POINTER(BsxChunks), c_void_p, c_void_p,
                             c_void_p, c_size_t, c_void_p]),
    ("bsx_attn_fwd_noalloc", c_int, [POINTER(BsxShape), c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_void_p, c_void_p, POINTER(BsxChunks), c_void_p,
                                     c_void_p, c_void_p]),
    ("bsx_lse_merge", c_int, [c_int32, c_int64, c_int32, c_void_p, c_void_p, c_int32, c_void_p,
                              c_void_p, c_void_p]),
    ("bsx_bwd_workspace", c_size_t, [POINTER(BsxShape), POINTER(BsxChunks)]),
    ("bsx_attn_bwd", c_int, [POINTER(BsxShape), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                             c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, POINTER(BsxChunks),
                             c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                             c_size_t, c_void_p]),
]

_lock = threading.Lock()
_lib = None


def _open() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        # Nothing built yet: build it (hipcc for gfx950); failures propagate.
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    for name, res, args in _SIGNATURES:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                _lib = _open()
    return _lib


def check(status: int) -> None:
    if status != BSX_OK:
        L = lib()
        name = L.bsx_status_string(status).decode()
        msg = L.bsx_last_error().decode()
        raise BsxError(status, f"{name}: {msg}")
