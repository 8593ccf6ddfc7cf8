"""ctypes view of ``libsplash.so`` (the C ABI declared in include/splash.h).

Only argument marshalling lives here.  The library is loaded on first use;
if it has not been built the import of an entry point raises, there is no
fallback implementation.
"""

from __future__ import annotations

import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsplash.so")

SPLASH_OK = 0
STATUS_NAMES = {
    0: "SPLASH_OK", 1: "SPLASH_EINVAL", 2: "SPLASH_ESHAPE", 3: "SPLASH_EDTYPE",
    4: "SPLASH_EUNSUPPORTED", 5: "SPLASH_ENOMEM", 6: "SPLASH_EHIP",
    7: "SPLASH_EINTERNAL",
}
SPLASH_F32 = 0
SPLASH_BF16 = 1
SPLASH_MASK_COMPUTED = 0
SPLASH_MASK_STORED = 1

# Every symbol include/splash.h declares.
EXPORTED = ("splash_version", "splash_last_error", "attn_mask_compile",
            "splash_fwd_tile", "splash_fwd_tiles", "splash_attn_fwd",
            "splash_split_workspace_bytes", "splash_attn_fwd_split",
            "splash_attn_fwd_split_noalloc", "attn_mask_columns", "attn_mask_column_order",
            "splash_bwd_tile", "splash_attn_bwd", "splash_clock_probe",
            "splash_realtime_khz")
SPLASH_MAX_SPLIT = 64
SPLASH_STATIC_SCRATCH_BYTES = 16 << 20

c_i32 = ctypes.c_int32
c_ptr = ctypes.c_void_p


class MaskDesc(ctypes.Structure):
    _fields_ = [("L_q", c_i32), ("L_kv", c_i32), ("block_q", c_i32),
                ("block_kv", c_i32), ("causal", c_i32), ("window_left", c_i32),
                ("window_right", c_i32), ("seg_q", c_ptr), ("seg_kv", c_ptr),
                ("q_offset", c_i32)]


class MaskSizes(ctypes.Structure):
    _fields_ = [("n_q_blocks", c_i32), ("n_kv_blocks", c_i32),
                ("n_active", c_i32), ("n_partial", c_i32), ("n_patterns", c_i32)]


class MaskTablesC(ctypes.Structure):
    _fields_ = [("block_mask", c_ptr), ("active_rows", c_ptr),
                ("active_cols", c_ptr), ("block_code", c_ptr),
                ("mask_next", c_ptr), ("bounds", c_ptr), ("row_ptr", c_ptr),
                ("row_order", c_ptr), ("partial_mask_blocks", c_ptr)]


class FwdArgs(ctypes.Structure):
    _fields_ = [("dtype", c_i32), ("B", c_i32), ("Hq", c_i32), ("Hkv", c_i32),
                ("L", c_i32), ("d_qk", c_i32), ("d_v", c_i32),
                ("q", c_ptr), ("k", c_ptr), ("v", c_ptr), ("o", c_ptr),
                ("lse", c_ptr),
                ("causal", c_i32), ("window_left", c_i32), ("window_right", c_i32),
                ("seg_q", c_ptr), ("seg_kv", c_ptr),
                ("block_q", c_i32), ("block_kv", c_i32), ("n_q_blocks", c_i32),
                ("n_active", c_i32), ("n_patterns", c_i32),
                ("row_ptr", c_ptr), ("row_order", c_ptr), ("active_cols", c_ptr),
                ("block_code", c_ptr), ("mask_next", c_ptr),
                ("partial_mask_blocks", c_ptr),
                ("mask_mode", c_i32), ("scale", ctypes.c_float),
                ("soft_cap", ctypes.c_float),
                ("use_max_logit", c_i32), ("max_logit", ctypes.c_float),
                ("L_kv", c_i32), ("q_offset", c_i32)]


class BwdArgs(ctypes.Structure):
    _fields_ = [("dtype", c_i32), ("B", c_i32), ("Hq", c_i32), ("Hkv", c_i32),
                ("L", c_i32), ("L_kv", c_i32), ("q_offset", c_i32),
                ("d_qk", c_i32), ("d_v", c_i32),
                ("q", c_ptr), ("k", c_ptr), ("v", c_ptr), ("o", c_ptr), ("lse", c_ptr),
                ("dout", c_ptr), ("dq", c_ptr), ("dk", c_ptr), ("dv", c_ptr),
                ("delta", c_ptr),
                ("causal", c_i32), ("window_left", c_i32), ("window_right", c_i32),
                ("seg_q", c_ptr), ("seg_kv", c_ptr),
                ("block_q", c_i32), ("block_kv", c_i32), ("n_q_blocks", c_i32),
                ("n_kv_blocks", c_i32), ("n_active", c_i32),
                ("row_ptr", c_ptr), ("row_order", c_ptr), ("active_cols", c_ptr),
                ("col_ptr", c_ptr), ("col_rows", c_ptr), ("col_order", c_ptr),
                ("scale", ctypes.c_float), ("soft_cap", ctypes.c_float)]


class SplashError(RuntimeError):
    """A non-zero status from the library, with its message."""

    def __init__(self, code: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {message}")
        self.code = code


_lock = threading.Lock()
_lib = None


def load():
    """Load libsplash.so (once).  Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m block_sparse_flash_amd.build` (no fallback path exists)")
        lib = ctypes.CDLL(LIB_PATH)
        lib.splash_version.restype = ctypes.c_int
        lib.splash_version.argtypes = []
        lib.splash_last_error.restype = ctypes.c_char_p
        lib.splash_last_error.argtypes = []
        lib.attn_mask_compile.restype = ctypes.c_int
        lib.attn_mask_compile.argtypes = [ctypes.POINTER(MaskDesc),
                                          ctypes.POINTER(MaskSizes),
                                          ctypes.POINTER(MaskTablesC)]
        lib.splash_fwd_tile.restype = ctypes.c_int
        lib.splash_fwd_tile.argtypes = [c_i32, c_i32, c_i32,
                                        ctypes.POINTER(c_i32), ctypes.POINTER(c_i32)]
        lib.splash_fwd_tiles.restype = ctypes.c_int
        lib.splash_fwd_tiles.argtypes = [c_i32, c_i32, c_i32, c_ptr, c_ptr, c_i32,
                                         ctypes.POINTER(c_i32)]
        lib.splash_bwd_tile.restype = ctypes.c_int
        lib.splash_bwd_tile.argtypes = [c_i32, c_i32, c_i32,
                                        ctypes.POINTER(c_i32), ctypes.POINTER(c_i32)]
        lib.splash_attn_fwd.restype = ctypes.c_int
        lib.splash_attn_fwd.argtypes = [ctypes.POINTER(FwdArgs), c_ptr]
        lib.splash_split_workspace_bytes.restype = ctypes.c_int
        lib.splash_split_workspace_bytes.argtypes = [c_i32, c_i32, c_i32, c_i32, c_i32,
                                                     ctypes.POINTER(ctypes.c_int64)]
        lib.splash_attn_fwd_split.restype = ctypes.c_int
        lib.splash_attn_fwd_split.argtypes = [ctypes.POINTER(FwdArgs), c_i32, c_ptr,
                                              ctypes.c_int64, c_ptr]
        lib.splash_attn_fwd_split_noalloc.restype = ctypes.c_int
        lib.splash_attn_fwd_split_noalloc.argtypes = [ctypes.POINTER(FwdArgs), c_i32, c_ptr]
        lib.attn_mask_columns.restype = ctypes.c_int
        lib.attn_mask_columns.argtypes = [c_i32, c_i32, c_i32, c_ptr, c_ptr, c_ptr, c_ptr, c_ptr]
        lib.attn_mask_column_order.restype = ctypes.c_int
        lib.attn_mask_column_order.argtypes = [c_i32, c_ptr, c_ptr]
        lib.splash_attn_bwd.restype = ctypes.c_int
        lib.splash_attn_bwd.argtypes = [ctypes.POINTER(BwdArgs), c_ptr]
        lib.splash_clock_probe.restype = ctypes.c_int
        lib.splash_clock_probe.argtypes = [c_ptr, c_i32, c_ptr]
        lib.splash_realtime_khz.restype = ctypes.c_int
        lib.splash_realtime_khz.argtypes = [ctypes.POINTER(c_i32)]
        _lib = lib
        return lib


def check(code: int):
    if code != SPLASH_OK:
        msg = load().splash_last_error()
        raise SplashError(code, msg.decode() if msg else "")
