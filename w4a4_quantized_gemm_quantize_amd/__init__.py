"""W4A4 group-quantized GEMM, MXFP4 GEMM and NVFP4 GEMM for MI355X (gfx950).

The compute lives in ``libw4a4.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/w4a4.h``). The Python side only marshals arguments; the
tensor-level entry points (same names as the C ABI) are in :mod:`.ops` and are
re-exported here on first use.
"""
_OPS = (
    "w4a4_quantize_act", "w4a4_pack_weight", "w4a4_gemm", "w4a4_gemm_splitk", "w4a4_gemm_debug_partials",
    "mxfp4_quantize", "mxfp4_quantize_residual", "mxfp4_quantize_append_copy",
    "mxfp4_gemm", "mxfp4_gemm_debug_partials",
    "nvfp4_global_scale", "nvfp4_quantize", "nvfp4_gemm", "nvfp4_gemm_debug_partials",
)


def __getattr__(name):
    if name in _OPS:
        from . import ops
        return getattr(ops, name)
    raise AttributeError(name)
