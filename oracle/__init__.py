"""CPU oracle for W4A4 group-quantized GEMM and the MXFP4 and NVFP4 variants.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or run anything in this directory. The
HIP library never calls it, shares no code with it and must fail loudly, not
fall back here, when its own build is missing.

The oracle is plain C++ (``orc.cpp``, built by ``python -m oracle.build`` with
-O2 -ffp-contract=off into ``liborc.so``): slow, unfused, obviously correct,
threaded over rows with std::thread. Floating point that decides an integer
(the INT4 codes, the NVFP4 scales and codes) is IEEE binary32, the precision
the GPU kernel takes the same decision in; sums of group terms are binary64.
The Python modules here only marshal numpy arrays (``int4``, ``mxfp4``,
``nvfp4``) and place codes and scales in the documented storage layouts
(``layout``: byte permutations, no arithmetic).

Pins (tests that tie each function to something other than itself) live in
``tests/test_oracle_*.py``. Every function here is pinned; none is "parity
unpinned".
"""
from . import _native  # noqa: F401
from .int4 import (  # noqa: F401
    int4_quantize,
    int4_dequantize,
    w4a4_block_partials,
    w4a4_gemm,
    w4a4_gemm_rows,
)
from .layout import (  # noqa: F401
    pack_nibbles,
    unpack_nibbles_unsigned,
    pack_int4_twos,
    unpack_int4_twos,
    pack_int4,
    unpack_int4,
    int4_sign_bits,
    group_major,
    e8m0_panel_offsets,
    e4m3_panel_offsets,
    to_panels,
    from_panels,
)
from .mxfp4 import (  # noqa: F401
    E2M1_VALUES,
    e2m1_decode,
    mxfp4_quantize,
    mxfp4_quantize_residual,
    mxfp4_quantize_residual_tied,
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


def set_threads(n: int) -> None:
    """Worker threads of every oracle call (0: every core this process may use)."""
    _native.threads = int(n)


def cores() -> int:
    """Threads an oracle call uses now."""
    return _native.cores()
