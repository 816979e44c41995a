"""ctypes binding of libw4a4.so (the C ABI declared in include/w4a4.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the ABI. PyTorch supplies device memory and the current stream.
There is no fallback: if the library is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libw4a4.so")

W4A4_OK = 0
STATUS_NAMES = {
    0: "W4A4_OK", 1: "W4A4_E_NULL", 2: "W4A4_E_SHAPE", 3: "W4A4_E_GROUP",
    4: "W4A4_E_ALIGN", 5: "W4A4_E_DTYPE", 6: "W4A4_E_HIP", 7: "W4A4_E_SCRATCH",
}
Y_F32 = 0
Y_F16 = 1

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32

# name -> argtypes, mirroring include/w4a4.h
SIGNATURES = {
    "w4a4_quantize_act": [_p, _i64, _i64, _i64, _i32, _p, _p, _p],
    "w4a4_pack_weight": [_p, _i64, _i64, _i32, _p, _p, _p],
    "w4a4_gemm": [_p, _p, _i32, _p, _p, _i32, _i64, _i64, _i64, _p, _i32, _i64, _p],
    "w4a4_gemm_debug_partials": [_p, _p, _i32, _p, _p, _i32, _i64, _i64, _i64,
                                 _i64, _i64, _i64, _i64, _p, _p],
    "w4a4_gemm_splitk": [_p, _p, _i32, _p, _p, _i32, _i64, _i64, _i64, _i32, _p, _i64,
                         _p, _i32, _i64, _p],
    "mxfp4_quantize": [_p, _i64, _i64, _i64, _p, _p, _p],
    "mxfp4_quantize_residual": [_p, _i64, _i64, _i64, _p, _p, _p],
    "mxfp4_quantize_append_copy": [_p, _i64, _i64, _i64, _p, _p, _p],
    "mxfp4_quantize_residual_tied": [_p, _i64, _i64, _i64, _p, _p, _p],
    "mxfp4_gemm": [_p, _p, _p, _p, _i64, _i64, _i64, _p, _i32, _i64, _p],
    "mxfp4_gemm_debug_partials": [_p, _p, _p, _p, _i64, _i64, _i64,
                                  _i64, _i64, _i64, _i64, _p, _p],
    "nvfp4_global_scale": [_p, _i64, _i64, _i64, _p, _p],
    "nvfp4_quantize": [_p, _i64, _i64, _i64, _p, _p, _p, _p],
    "nvfp4_gemm": [_p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _p, _i32, _i64, _p],
    "nvfp4_gemm_debug_partials": [_p, _p, _p, _p, _i64, _i64, _i64,
                                  _i64, _i64, _i64, _i64, _p, _p],
    "w4a4_gemm_splitk_noalloc": [_p, _p, _i32, _p, _p, _i32, _i64, _i64, _i64, _i32,
                                 _p, _i32, _i64, _p],
    "w4a4_linear_fused": [_p, _i64, _i64, _i64, _i32, _p, _p, _i32, _i64, _p, _i32, _i64, _p],
    "w4a4_repack_int4": [_p, _i64, _i64, _p, _p, _p],
    "w4a4_probe_mfma": [_i32, _i64, _p, _p],
    "w4a4_probe_hbm_read": [_p, _i64, _p, _p],
    "w4a4_probe_hbm_copy": [_p, _i64, _p, _p],
    "w4a4_unpack_int4": [_p, _i64, _i64, _p, _p],
    "w4a4_scales_to_group_major": [_p, _i64, _i64, _p, _p],
    "w4a4_scales_to_row_major": [_p, _i64, _i64, _p, _p],
    "mxfp4_scales_to_panels": [_p, _i64, _i64, _p, _p],
    "mxfp4_scales_to_rows": [_p, _i64, _i64, _p, _p],
    "nvfp4_scales_to_panels": [_p, _i64, _i64, _p, _p],
    "nvfp4_scales_to_rows": [_p, _i64, _i64, _p, _p],
}


class W4A4Error(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str = ""):
        self.status = status
        name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{fn} returned {name}" + (f": {detail}" if detail else ""))


_lib = None
_lock = threading.Lock()


def load_library() -> ctypes.CDLL:
    """Load libw4a4.so (once). Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m w4a4_quantized_gemm_quantize_amd.build)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, argtypes in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = argtypes
            fn.restype = ctypes.c_int
        lib.w4a4_status_str.argtypes = [ctypes.c_int]
        lib.w4a4_status_str.restype = ctypes.c_char_p
        lib.w4a4_gemm_splitk_workspace.argtypes = [_i64, _i64, _i64, _i32, _i32, _i32]
        lib.w4a4_gemm_splitk_workspace.restype = ctypes.c_int64
        lib.w4a4_linear_fused_supported.argtypes = [_i64, _i64, _i64, _i32, _i32]
        lib.w4a4_linear_fused_supported.restype = ctypes.c_int32
        lib.w4a4_probe_sink_bytes.argtypes = []
        lib.w4a4_probe_sink_bytes.restype = ctypes.c_int64
        lib.w4a4_probe_mfma_ops.argtypes = [_i32, _i64]
        lib.w4a4_probe_mfma_ops.restype = ctypes.c_int64
        lib.w4a4_gemm_splitk_noalloc_max_bytes.argtypes = []
        lib.w4a4_gemm_splitk_noalloc_max_bytes.restype = ctypes.c_int64
        _lib = lib
        return lib


def splitk_workspace_bytes(M: int, N: int, K: int, group_a: int, group_w: int, splits: int) -> int:
    """Bytes of workspace w4a4_gemm_splitk needs (0: it runs unsplit); raises on invalid arguments."""
    n = load_library().w4a4_gemm_splitk_workspace(M, N, K, group_a, group_w, splits)
    if n < 0:
        raise W4A4Error("w4a4_gemm_splitk_workspace", 2, "invalid arguments")
    return n


def call(name: str, *args) -> None:
    """Call an ABI entry point; raise W4A4Error on a non-OK status."""
    lib = load_library()
    st = getattr(lib, name)(*args)
    if st != W4A4_OK:
        raise W4A4Error(name, st, lib.w4a4_status_str(st).decode())


def status_of(name: str, *args) -> int:
    """Call an ABI entry point and return its raw status (for validation tests)."""
    return getattr(load_library(), name)(*args)
