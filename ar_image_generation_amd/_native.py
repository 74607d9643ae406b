"""ctypes view of libdiagattn.so (declared in include/diagattn.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation anywhere in this package.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; DIAGATTN_LIB names another build of the same sources
# (e.g. the host-AddressSanitizer one of build.py)
LIB_PATH = os.environ.get("DIAGATTN_LIB") or os.path.join(HERE, "libdiagattn.so")

c_i32, c_i64, c_f32, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p


class DaMask(ctypes.Structure):
    _fields_ = [("mode", c_i32), ("W", c_i32), ("B", c_i32), ("G", c_i32), ("causal", c_i32)]


class DaKvCache(ctypes.Structure):
    _fields_ = [("k", c_vp), ("v", c_vp), ("page_stride", c_i64), ("head_stride", c_i64),
                ("slot_stride", c_i64), ("page_size", c_i32), ("bt_stride", c_i32),
                ("block_table", c_vp), ("n_seq", c_i32), ("n_pages", c_i32), ("max_len", c_i32)]


# name -> (restype, argtypes); every symbol include/diagattn.h declares
SIGNATURES = {
    "da_version": (c_i32, []),
    "da_last_error": (ctypes.c_char_p, []),
    "da_keep_count": (c_i64, [ctypes.POINTER(DaMask), c_i32, c_i32, c_i32]),
    "da_keep_cap": (c_i64, [ctypes.POINTER(DaMask), c_i32, c_i32, c_i32]),
    "da_keepset_build": (ctypes.c_int, [ctypes.POINTER(DaMask), c_i32, c_vp, c_vp, c_i32, c_i32,
                                        c_vp, c_i32, c_vp, c_vp, c_i32, c_vp, c_vp, c_i32, c_vp,
                                        c_i64, c_vp, c_vp]),
    "da_decode_workspace_bytes": (c_i64, [c_i32, c_i32, c_i32, c_i32, c_i32]),
    "da_hbm_read_probe": (ctypes.c_int, [c_vp, c_i64, c_vp, c_i32, c_i32, c_vp]),
    "da_gather_read_probe": (ctypes.c_int, [c_vp, c_vp, c_vp, c_i64, c_i32, c_i64, c_vp, c_i32, c_i32, c_vp]),
    "da_prefill_tiles_bytes": (c_i64, [c_i32, c_i32]),
    "da_prefill_tiles_build": (ctypes.c_int, [ctypes.POINTER(DaMask), c_i32, c_i32, c_vp, c_vp,
                                              c_i64, c_vp]),
    "da_band_prefill_attn": (ctypes.c_int, [ctypes.POINTER(DaMask), ctypes.c_int, c_i32, c_i32, c_i32,
                                            c_i32, c_i32, c_vp, c_vp, c_vp, c_vp,
                                            ctypes.POINTER(c_i64), c_vp, c_vp, c_i64, c_f32, c_vp, c_vp]),
    "da_sparse_decode_attn": (ctypes.c_int, [c_vp, ctypes.c_int, c_i32, c_i32, c_i32, c_i32, c_f32,
                                             ctypes.POINTER(DaKvCache), c_vp, c_vp, c_vp, c_i32,
                                             c_i32, c_i32, c_vp, c_vp, c_vp, c_i64, c_vp]),
    "da_ring_pages": (c_i64, [ctypes.POINTER(DaMask), c_i32, c_i32, c_i32]),
    "da_ring_block_table": (ctypes.c_int, [ctypes.POINTER(DaMask), c_i32, c_vp, c_i32, c_i32, c_i32,
                                           c_i32, c_vp, c_vp]),
    "da_decode_scratch_bytes": (c_i64, []),
    "da_decode_schedule": (ctypes.c_int, [c_vp, c_i32, c_i32, c_i32, c_vp]),
    "da_sparse_decode_attn_masked_noalloc": (ctypes.c_int, [ctypes.POINTER(DaMask), c_vp, ctypes.c_int,
                                                            c_i32, c_i32, c_i32, c_i32, c_f32,
                                                            ctypes.POINTER(DaKvCache), c_vp, c_vp,
                                                            c_vp, c_vp, c_vp, c_vp, c_i32, c_i32,
                                                            c_vp, c_vp, c_vp, c_vp, c_vp]),
    "da_sparse_decode_attn_masked": (ctypes.c_int, [ctypes.POINTER(DaMask), c_vp, ctypes.c_int, c_i32,
                                                    c_i32, c_i32, c_i32, c_f32,
                                                    ctypes.POINTER(DaKvCache), c_vp, c_vp, c_vp,
                                                    c_vp, c_vp, c_vp,
                                                    c_i32, c_i32, c_vp, c_vp, c_vp, c_vp, c_vp,
                                                    c_i64, c_vp]),
}

_lib = None
_lock = threading.Lock()


class DiagAttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what} (status {status})")
        self.status = status


def load() -> ctypes.CDLL:
    """The loaded library; raises if it is not built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with "
                    "`python -m ar_image_generation_amd.build` (hipcc, gfx950)")
            lib = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                if not hasattr(lib, name):
                    continue
                f = getattr(lib, name)
                f.restype = res
                f.argtypes = args
            _lib = lib
    return _lib


def last_error() -> str:
    return load().da_last_error().decode()


def check(status: int, what: str) -> None:
    if status != 0:
        raise DiagAttnError(status, f"{what}: {last_error()}")
