"""CPU oracle for W4A4 group-quantized GEMM and the MXFP4 and NVFP4 variants.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or run anything in this directory. The
HIP library never calls it, shares no code with it and must fail loudly, not
fall back here, when its own build is missing.

The oracle is plain numpy: slow, unfused, obviously correct. Floating point that
decides an integer (the INT4 codes, the NVFP4 scales and codes) is done in IEEE
binary32, the precision the GPU kernel takes the same decision in; everything
else is float64. Each function
names the passage of the pages it follows and, where the pages are silent,
states the reading taken.

Pins (tests that tie each function to something other than itself) live in
``tests/test_oracle_*.py``. Every function here is pinned; none is "parity
unpinned".
"""
from .int4 import (  # noqa: F401
    int4_quantize,
    int4_dequantize,
    pack_nibbles,
    unpack_nibbles_unsigned,
    pack_int4,
    unpack_int4,
    int4_sign_bits,
    w4a4_block_partials,
    w4a4_gemm,
    w4a4_gemm_rows,
)
from .mxfp4 import (  # noqa: F401
    E2M1_VALUES,
    e2m1_decode,
    mxfp4_quantize,
    mxfp4_quantize_residual,
    mxfp4_append_copy,
    mxfp4_dequantize,
    mxfp4_block_partials,
    mxfp4_gemm,
)
from .nvfp4 import (  # noqa: F401
    e4m3_decode,
    e4m3_round,
    nvfp4_global_scale,
    nvfp4_quantize,
    nvfp4_dequantize,
    nvfp4_block_partials,
    nvfp4_gemm,
)
