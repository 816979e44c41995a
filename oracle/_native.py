"""ctypes loader of the C++ oracle (``liborc.so``, built from ``orc.cpp``).

TEST INFRASTRUCTURE ONLY. Argument marshalling between numpy arrays and the
oracle's C entry points; no arithmetic of the method is done here.
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liborc.so")

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int
_f32 = ctypes.c_float
_f64 = ctypes.c_double

_SIGS = {
    "orc_default_threads": ([], _i32),
    "orc_f16_to_f32": ([ctypes.c_uint16], _f32),
    "orc_f32_to_f16": ([_f32], ctypes.c_uint16),
    "orc_f16_to_f32_array": ([_p, _i64, _p], None),
    "orc_f32_to_f16_array": ([_p, _i64, _p], None),
    "orc_int4_quantize": ([_p, _i64, _i64, _i64, _p, _p, _i32], _i32),
    "orc_int4_dequantize": ([_p, _p, _i64, _i64, _i64, _p], None),
    "orc_w4a4_block_partials": ([_p, _p, _i64, _i64, _i64, _i64, _p, _i32], _i32),
    "orc_w4a4_gemm": ([_p, _p, _i64, _p, _p, _i64, _i64, _i64, _i64, _p, _p, _i32], _i32),
    "orc_e2m1_value": ([ctypes.c_uint8], _f64),
    "orc_mxfp4_quantize": ([_p, _i64, _i64, _p, _p, _i32], _i32),
    "orc_mxfp4_quantize_residual": ([_p, _i64, _i64, _p, _p, _i32], _i32),
    "orc_mxfp4_quantize_residual_tied": ([_p, _i64, _i64, _p, _p, _i32], _i32),
    "orc_mxfp4_dequantize": ([_p, _p, _i64, _i64, _p], None),
    "orc_fp4_block_partials": ([_p, _p, _i64, _i64, _i64, _i64, _p, _i32], _i32),
    "orc_mxfp4_gemm": ([_p, _p, _p, _p, _i64, _i64, _i64, _p, _p, _i32], _i32),
    "orc_e4m3_value": ([ctypes.c_uint8], _f64),
    "orc_e4m3_round": ([_f64], ctypes.c_uint8),
    "orc_nvfp4_global_scale": ([_p, _i64, _p], _i32),
    "orc_nvfp4_quantize": ([_p, _i64, _i64, _f32, _p, _p, _i32], _i32),
    "orc_nvfp4_gemm": ([_p, _p, _f32, _p, _p, _f32, _i64, _i64, _i64, _p, _p, _i32], _i32),
    "orc_nvfp4_dequantize": ([_p, _p, _f32, _i64, _i64, _p], None),
}

_ERRORS = {
    1: "NaN/Inf inputs are outside the quantizer's contract",
    2: "unsupported shape or group size",
    3: "a partial sum does not fit int32",
    4: "the global scale must be finite and >= 0",
}

_lib = None
_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """The loaded oracle library; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB):
                # test infrastructure: build it on first use (g++, a few seconds)
                from .build import build
                build()
            handle = ctypes.CDLL(LIB)
            for name, (args, res) in _SIGS.items():
                fn = getattr(handle, name)
                fn.argtypes = args
                fn.restype = res
            _lib = handle
        return _lib


def check(status: int) -> None:
    if status:
        raise ValueError(_ERRORS.get(status, f"oracle status {status}"))


def ptr(a: np.ndarray) -> int:
    """Address of a C-contiguous array's data."""
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# Worker threads of every oracle call (0: the cores this process may run on).
threads = 0


def cores() -> int:
    """Threads an oracle call with ``threads == 0`` uses."""
    return threads if threads > 0 else lib().orc_default_threads()
