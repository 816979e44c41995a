"""W4A4 group-quantized GEMM and MXFP4 GEMM for MI355X (gfx950).

The compute lives in ``libw4a4.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/w4a4.h``). The Python side only marshals arguments.
"""
