"""ctypes declarations of liboscar's C ABI (include/oscar.h).

torch is imported before the library is opened so that liboscar binds to the
HIP runtime torch already loaded (one runtime per process).  A missing
library raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must precede loading liboscar.so)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liboscar.so")

OSCAR_OK = 0
OSCAR_EINVAL = -1
OSCAR_EUNSUPPORTED = -2
OSCAR_EWORKSPACE = -3
OSCAR_EHIP = -4
OSCAR_ENODEV = -5
STATUS_BAD_PAGE = 1
STATUS_BAD_LEN = 2

c_p = ctypes.c_void_p


class LayerCacheC(ctypes.Structure):
    _fields_ = [("n_kv_heads", ctypes.c_int32),
                ("group", ctypes.c_int32),
                ("hist", c_p),
                ("n_hist_pages", ctypes.c_int64),
                ("bf16", c_p),
                ("n_bf16_pages", ctypes.c_int64),
                ("hist_pt", c_p),
                ("hist_pt_stride", ctypes.c_int32),
                ("bf16_pt", c_p),
                ("status", c_p),
                ("code_bits", ctypes.c_int32)]


MAX_HEAD_ROTATIONS = 32  # OSCAR_MAX_HEAD_ROTATIONS


class RotationC(ctypes.Structure):
    _fields_ = [("forms", c_p), ("clip", ctypes.c_float), ("n_heads", ctypes.c_int32),
                ("head_clips", ctypes.POINTER(ctypes.c_float))]


# (name, restype, argtypes) of every exported function
SIGNATURES = [
    ("oscar_last_error", ctypes.c_char_p, []),
    ("oscar_version", ctypes.c_char_p, []),
    ("oscar_hist_block_bytes", ctypes.c_size_t, [ctypes.c_int32]),
    ("oscar_hist_block_bytes_bits", ctypes.c_size_t, [ctypes.c_int32, ctypes.c_int32]),
    ("oscar_rotation_bytes", ctypes.c_size_t, []),
    ("oscar_prepare_rotation", ctypes.c_int, [c_p, c_p, c_p]),
    ("oscar_calibrate_workspace_bytes", ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]),
    ("oscar_calib_accumulate_workspace_bytes", ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]),
    ("oscar_calib_rotations_workspace_bytes", ctypes.c_size_t, []),
    ("oscar_clip_threshold_workspace_bytes", ctypes.c_size_t, [ctypes.c_int64]),
    ("oscar_calibrate_rotation", ctypes.c_int,
     [c_p, c_p, c_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_double,
      c_p, c_p, c_p, c_p, c_p, ctypes.c_size_t, c_p]),
    ("oscar_calib_accumulate", ctypes.c_int,
     [c_p, c_p, c_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, c_p, c_p, ctypes.c_size_t, c_p]),
    ("oscar_calib_accumulate_heads", ctypes.c_int,
     [c_p, c_p, c_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, c_p, c_p, ctypes.c_size_t, c_p]),
    ("oscar_calib_rotations", ctypes.c_int, [c_p, ctypes.c_double, c_p, c_p, c_p, ctypes.c_size_t, c_p]),
    ("oscar_clip_threshold", ctypes.c_int,
     [c_p, ctypes.c_int64, c_p, ctypes.c_double, c_p, c_p, ctypes.c_size_t, c_p]),
    ("oscar_write_kv", ctypes.c_int,
     [ctypes.POINTER(LayerCacheC), ctypes.POINTER(RotationC), ctypes.POINTER(RotationC),
      c_p, c_p, c_p, c_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, c_p]),
    ("oscar_decode_workspace_bytes", ctypes.c_size_t,
     [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]),
    ("oscar_decode_attn", ctypes.c_int,
     [ctypes.POINTER(LayerCacheC), ctypes.POINTER(RotationC), ctypes.POINTER(RotationC),
      c_p, ctypes.c_int32, c_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, c_p,
      c_p, ctypes.c_size_t, c_p]),
    ("oscar_decode_step", ctypes.c_int,
     [ctypes.POINTER(LayerCacheC), ctypes.POINTER(RotationC), ctypes.POINTER(RotationC),
      c_p, c_p, c_p, c_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, c_p,
      c_p, ctypes.c_size_t, c_p]),
    ("oscar_extend_attn", ctypes.c_int,
     [ctypes.POINTER(LayerCacheC), ctypes.POINTER(RotationC), ctypes.POINTER(RotationC),
      c_p, ctypes.c_int32, c_p, c_p, c_p, c_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
      ctypes.c_float, c_p, c_p]),
    ("oscar_profile_events", ctypes.c_int, [c_p, c_p]),
    ("oscar_decode_noalloc_max_bytes", ctypes.c_size_t, []),
    ("oscar_decode_attn_noalloc", ctypes.c_int,
     [ctypes.POINTER(LayerCacheC), ctypes.POINTER(RotationC), ctypes.POINTER(RotationC),
      c_p, ctypes.c_int32, c_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, c_p, c_p]),
    ("oscar_read_probe", ctypes.c_int,
     [c_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, c_p, c_p, c_p]),
    ("oscar_bf16_decode_workspace_bytes", ctypes.c_size_t,
     [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]),
    ("oscar_bf16_paged_decode", ctypes.c_int,
     [c_p, c_p, ctypes.c_int64, c_p, ctypes.c_int32, c_p, ctypes.c_int32, ctypes.c_int32,
      ctypes.c_int32, ctypes.c_int32, ctypes.c_float, c_p, c_p, c_p, ctypes.c_size_t, c_p]),
]

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Open liboscar.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"liboscar.so not built at {path}; run `python bit_rotated_kv_oscar_amd/build.py`")
    lib = ctypes.CDLL(path)
    for name, res, args in SIGNATURES:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class OscarError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"liboscar error {code}: {msg}")
        self.code = code


def check(rc: int) -> None:
    if rc != OSCAR_OK:
        raise OscarError(rc, load().oscar_last_error().decode())
