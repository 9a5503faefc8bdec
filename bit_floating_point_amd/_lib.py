"""ctypes mirror of include/fp4.h and the loader of libfp4.so.

The library is built in-tree (``python -m bit_floating_point_amd.build``).  If it is
missing, importing this module raises: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfp4.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "fp4.h")

FP4_OK, FP4_ERR_INVALID_ARG, FP4_ERR_UNSUPPORTED, FP4_ERR_ALIGNMENT, FP4_ERR_WORKSPACE, FP4_ERR_HIP = range(6)
FP4_F32, FP4_BF16, FP4_F16, FP4_PACKED = 0, 1, 2, 3
FP4_GRID_MINIFLOAT, FP4_GRID_LUT16, FP4_GRID_TWO_MODE = 0, 1, 2
FP4_SCALE_TENSOR, FP4_SCALE_ROW, FP4_SCALE_GROUP = 0, 1, 2
FP4_REDUCE_TENSOR, FP4_REDUCE_COLUMN, FP4_REDUCE_ROW_GROUP = 0, 1, 2


class fp4_grid(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("e", ctypes.c_int32), ("m", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("lut", ctypes.c_float * 16)]


class fp4_gran(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("group", ctypes.c_int32), ("scale_dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class fp4_search_result(ctypes.Structure):
    _fields_ = [("e", ctypes.c_int32), ("m", ctypes.c_int32), ("clip_index", ctypes.c_int32),
                ("format_index", ctypes.c_int32), ("clip", ctypes.c_float), ("scale", ctypes.c_float),
                ("amax", ctypes.c_float), ("reserved", ctypes.c_float), ("bias", ctypes.c_double),
                ("mse", ctypes.c_double), ("mse_runner_up", ctypes.c_double)]


class fp4_gemm_desc(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("a_kind", ctypes.c_int32), ("a_scale_mode", ctypes.c_int32),
                ("a", ctypes.c_void_p), ("lda", ctypes.c_int64), ("a_grid", fp4_grid),
                ("a_scale", ctypes.c_void_p),
                ("w", ctypes.c_void_p), ("ldw", ctypes.c_int64), ("w_grid", fp4_grid),
                ("w_gran", fp4_gran), ("w_scales", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("ldy", ctypes.c_int64), ("y_dtype", ctypes.c_int32),
                ("reserved1", ctypes.c_int32)]



class fp4_swiglu_desc(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("a", ctypes.c_void_p), ("lda", ctypes.c_int64), ("a_scale", ctypes.c_void_p),
                ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("ldw", ctypes.c_int64),
                ("s_gate", ctypes.c_void_p), ("s_up", ctypes.c_void_p),
                ("out_scale", ctypes.c_void_p), ("out_shift", ctypes.c_void_p),
                ("h_packed", ctypes.c_void_p), ("ldh", ctypes.c_int64)]

# exported symbol -> (restype, argtypes)
P, I32, I64, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
SIGNATURES = {
    "fp4_status_string": (ctypes.c_char_p, [I32]),
    "fp4_last_error": (ctypes.c_char_p, []),
    "fp4_calibrate": (I32, [P, I32, I64, I64, I64, I32, I32, I64, P, P]),
    "fp4_quantize_pack": (I32, [P, I32, I64, I64, I64, fp4_grid, fp4_gran, P, P, P, P, I64, P, P]),
    "fp4_dequantize": (I32, [P, I64, I64, I64, fp4_grid, fp4_gran, P, P, P, I64, P]),
    "fp4_preshift_weights": (I32, [P, I64, I64, I64, P, fp4_grid, fp4_grid, fp4_gran, P, P, P, I64, P, P]),
    "fp4_search_workspace_size": (ctypes.c_size_t, [I64, I64, I32, I32]),
    "fp4_search_format": (I32, [P, I64, I64, P, I32, I32, F32, F32, P, P, P, ctypes.c_size_t, P]),
    "fp4_search_format_static": (I32, [P, I64, I64, P, I32, I32, F32, F32, P, P, P]),
    "fp4_search_activations": (I32, [P, I32, I64, I64, I64, I32, I64, P, I32, I32, F32, F32, P, P, I64, P,
                                     ctypes.c_size_t, P]),
    "fp4_gemm": (I32, [ctypes.POINTER(fp4_gemm_desc), P]),
    "fp4_gemm_swiglu_quant": (I32, [ctypes.POINTER(fp4_swiglu_desc), P]),
    "fp4_set_split_limit": (I32, [I64]),
    "fp4_nf4_grid": (I32, [ctypes.POINTER(fp4_grid)]),
}


class FP4Error(RuntimeError):
    def __init__(self, status: int, func: str, msg: str):
        super().__init__(f"{func}: {msg} ({status})")
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m bit_floating_point_amd.build` "
                          "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_LIB = None


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        _LIB = load()
    return _LIB


def check(status: int, func: str) -> None:
    if status != FP4_OK:
        L = lib()
        raise FP4Error(status, func, L.fp4_last_error().decode() or L.fp4_status_string(status).decode())
