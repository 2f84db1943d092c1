"""ctypes view of libw4a4.so: the C ABI declared in include/w4a4.h, nothing more.

Loading fails loudly when the library has not been built: there is no other
implementation behind these names.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libw4a4.so")

W4A4_OK, W4A4_ERR_NULL, W4A4_ERR_SHAPE, W4A4_ERR_ALIGN, W4A4_ERR_MODE, W4A4_ERR_DEVICE = range(6)
W4A4_HAD_FULL, W4A4_HAD_128 = 0, 128
W4A4_ACT_SYM_TOKEN, W4A4_ACT_ASYM_G128 = 0, 1
STATUS_NAMES = {0: "W4A4_OK", 1: "W4A4_ERR_NULL", 2: "W4A4_ERR_SHAPE", 3: "W4A4_ERR_ALIGN",
                4: "W4A4_ERR_MODE", 5: "W4A4_ERR_DEVICE"}

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32

SIGNATURES = {
    "rotate_quant_act": [_vp, _i64, _i64, _i64, _i32, _vp, _i32, _vp, _vp, _vp, _vp],
    "quant_weight_offline": [_vp, _i64, _i64, _i64, _i32, _vp, _vp, _vp, _vp, _vp],
    "w4a4_gemm": [_vp, _vp, _vp, _i32, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _i64, _vp],
    "kv_rotate_quant4": [_vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp],
    "w4a4_time_next_launch": [_vp, _vp],
    "kv4_attention_decode": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, ctypes.c_float,
                             _vp, _vp, _vp],
    "rotate_quant_mxfp4": [_vp, _i64, _i64, _i64, _i32, _vp, _vp, _vp, _vp],
    "w4a4_decode_fused": [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _i64, _vp, _i64, _vp],
    "mxfp4_gemm": [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp, _i64, _vp],
    "kv4_attention_decode_ws": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, ctypes.c_float,
                                _vp, _vp, _vp, _i64, _vp],
    "kv4_attention_decode_noalloc": [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, ctypes.c_float,
                                     _vp, _vp, _vp],
}
# entry points that return a value other than a status
SIZE_FUNCS = {"kv4_attention_workspace_bytes": [_i64, _i64, _i64]}

_lib = None


def load() -> ctypes.CDLL:
    """Load the built library (once).  Raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it first "
                              "(python -m rotation_w4a4_quantization_amd.build)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, args in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        for name, args in SIZE_FUNCS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int64
        lib.w4a4_last_error.argtypes = []
        lib.w4a4_last_error.restype = ctypes.c_char_p
        lib.w4a4_abi_version.argtypes = []
        lib.w4a4_abi_version.restype = ctypes.c_int32
        _lib = lib
    return _lib


def last_error() -> str:
    return load().w4a4_last_error().decode()


def call(name: str, *args) -> int:
    """Call one entry point with raw integers / pointers; returns the status."""
    return getattr(load(), name)(*args)
