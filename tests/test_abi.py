"""The C ABI (CPU only): libw4a4.so loads, exports every function that
include/w4a4.h declares with the argument count the binding uses, and rejects
bad arguments with the documented status before touching the GPU.

The validation calls below return before any HIP call, so they run without a
GPU. Pointers passed are fake but never dereferenced on those paths.
"""
import ctypes
import glob
import os
import re

import pytest

from w4a4_quantized_gemm_quantize_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

OK, E_NULL, E_SHAPE, E_GROUP, E_ALIGN, E_DTYPE = 0, 1, 2, 3, 4, 5
P = 0x10000          # a fake, 64 KiB-aligned "device pointer"


def header_functions():
    text = "\n".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    out = {}
    for m in re.finditer(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(\w+)\s*\(([^;]*?)\)\s*;", text, flags=re.M | re.S):
        name, args = m.group(1), m.group(2)
        out[name] = 0 if args.strip() in ("", "void") else args.count(",") + 1
    return out


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libw4a4.so is not built (python -m w4a4_quantized_gemm_quantize_amd.build)")
    return _lib.load_library()


def test_every_declared_symbol_is_exported(lib):
    decls = header_functions()
    assert set(decls) >= set(_lib.SIGNATURES) | {"w4a4_status_str"}
    for name, nargs in decls.items():
        assert hasattr(lib, name), name
        if name in _lib.SIGNATURES:
            assert len(_lib.SIGNATURES[name]) == nargs, name


def test_status_strings(lib):
    for st in range(8):
        s = lib.w4a4_status_str(st)
        assert s and s != b"unknown status"
    assert lib.w4a4_status_str(99) == b"unknown status"


def q(*a):
    return _lib.status_of("w4a4_quantize_act", *a)


def test_quantize_act_validation(lib):
    M, K = 4, 256
    assert q(P, -1, K, K, 128, P, P, None) == E_SHAPE
    assert q(P, M, 0, K, 128, P, P, None) == E_SHAPE
    assert q(P, M, 260, 264, 128, P, P, None) == E_SHAPE      # K % 16 != 0 (260 % 16 = 4)
    assert q(P, M, 264, 264, 264, P, P, None) == E_SHAPE      # per token, but 264 % 16 = 8
    assert q(P, M, K, K - 8, 128, P, P, None) == E_SHAPE     # ldx < K
    assert q(P, M, K, K, 96, P, P, None) == E_GROUP
    assert q(P, M, K, K, 512, P, P, None) == E_GROUP         # 512 does not divide 256
    assert q(P, M, 384, 384, 256, P, P, None) == E_GROUP
    assert q(P, M, K, K + 4, 128, P, P, None) == E_ALIGN     # ldx % 8
    assert q(P, 0, K, K, 128, None, None, None) == OK        # empty: no-op
    assert q(None, M, K, K, 128, P, P, None) == E_NULL
    assert q(P, M, K, K, 128, None, P, None) == E_NULL
    assert q(P + 8, M, K, K, 128, P, P, None) == E_ALIGN
    assert q(P, M, K, K, 128, P + 2, P, None) == E_ALIGN
    assert q(P, M, K, K, 128, P + 4, P, None) == E_ALIGN        # 8-byte packed units
    assert _lib.status_of("w4a4_pack_weight", P, M, K, 100, P, P, None) == E_GROUP
    assert _lib.status_of("w4a4_pack_weight", None, M, K, 128, P, P, None) == E_NULL


def g(*a):
    return _lib.status_of("w4a4_gemm", *a)


def test_gemm_validation(lib):
    M, N, K = 16, 32, 256
    assert g(P, P, 128, P, P, 128, M, N, 200, P, 0, N, None) == E_SHAPE       # K % 128
    assert g(P, P, 128, P, P, 128, -1, N, K, P, 0, N, None) == E_SHAPE
    assert g(P, P, 96, P, P, 128, M, N, K, P, 0, N, None) == E_GROUP
    assert g(P, P, 128, P, P, 192, M, N, 384, P, 0, N, None) == E_GROUP       # 192 not a power of two
    assert g(P, P, 256, P, P, 384, M, N, 768, P, 0, N, None) == E_GROUP       # not nested
    assert g(P, P, 512, P, P, 128, M, N, K, P, 0, N, None) == E_GROUP         # 512 !| 256
    # the finer group bounds the fp32 partials: 49 g must stay below 2^24
    big = 1 << 19
    assert g(P, P, big, P, P, big, M, N, big, P, 0, N, None) == E_GROUP       # per token, g = 2^19
    assert g(P, P, 128, P, P, 128, M, N, (1 << 23) + 128, P, 0, N, None) == E_SHAPE   # 32-bit tile offsets
    assert g(P, P, 128, P, P, 128, M, N, 1 << 24, P, 0, N, None) == E_SHAPE
    assert g(P, P, 128, P, P, 128, 0, N, 1 << 23, None, 0, N, None) == OK             # the longest K
    assert _lib.load_library().w4a4_gemm_splitk_workspace(M, N, 1 << 24, 128, 128, 0) == -1
    assert g(P, P, 128, P, P, 128, 0, N, K, None, 0, N, None) == OK           # empty
    assert g(P, P, 128, P, P, 128, M, 0, K, None, 0, 0, None) == OK
    assert g(None, P, 128, P, P, 128, M, N, K, P, 0, N, None) == E_NULL
    assert g(P, P, 128, P, None, 128, M, N, K, P, 0, N, None) == E_NULL
    assert g(P + 4, P, 128, P, P, 128, M, N, K, P, 0, N, None) == E_ALIGN
    assert g(P, P + 1, 128, P, P, 128, M, N, K, P, 0, N, None) == E_ALIGN
    assert g(P, P, 128, P, P, 128, M, N, K, P, 7, N, None) == E_DTYPE
    assert g(P, P, 128, P, P, 128, M, N, K, P, 0, N - 1, None) == E_SHAPE     # ldy < N
    assert g(P, P, 128, P, P, 128, M, N, K, None, 0, N, None) == E_NULL
    assert g(P, P, 128, P, P, 128, M, N, K, P + 2, 0, N, None) == E_ALIGN     # f32 y
    dp = lambda *a: _lib.status_of("w4a4_gemm_debug_partials", *a)
    assert dp(P, P, 128, P, P, 128, M, N, K, 0, M + 1, 0, N, P, None) == E_SHAPE
    assert dp(P, P, 128, P, P, 128, M, N, K, 5, 0, 0, N, P, None) == E_SHAPE
    assert dp(P, P, 128, P, P, 128, M, N, K, 0, M, -1, 4, P, None) == E_SHAPE
    assert dp(P, P, 128, P, P, 128, M, N, K, 0, M, 0, N, None, None) == E_NULL


def test_mxfp4_validation(lib):
    mq = lambda *a: _lib.status_of("mxfp4_quantize", *a)
    assert mq(P, 4, 48, 48, P, P, None) == E_SHAPE
    assert mq(P, 4, 64, 60, P, P, None) == E_SHAPE
    assert mq(P, 4, 64, 68, P, P, None) == E_ALIGN
    assert mq(P, 0, 64, 64, None, None, None) == OK
    assert mq(None, 4, 64, 64, P, P, None) == E_NULL
    for fn in ("mxfp4_quantize_residual", "mxfp4_quantize_append_copy", "mxfp4_quantize_residual_tied"):
        r = lambda *a: _lib.status_of(fn, *a)
        assert r(P, 4, 48, 48, P, P, None) == E_SHAPE
        assert r(P, 4, 64, 68, P, P, None) == E_ALIGN
        assert r(P, 0, 64, 64, None, None, None) == OK
        assert r(P, 4, 64, 64, None, P, None) == E_NULL
        assert r(P, 4, 64, 64, P + 2, P, None) == E_ALIGN
    mg = lambda *a: _lib.status_of("mxfp4_gemm", *a)
    assert mg(P, P, P, P, 4, 4, 96, P, 0, 4, None) == E_SHAPE
    assert mg(P, P, P, P, 4, 4, 128, P, 2, 4, None) == E_DTYPE
    assert mg(P, P + 2, P, P, 4, 4, 128, P, 0, 4, None) == E_ALIGN
    assert mg(P, P, P, None, 4, 4, 128, P, 0, 4, None) == E_NULL
    assert mg(P, P, P, P, 0, 4, 128, None, 0, 4, None) == OK
    assert mg(P, P, P, P, 4, 4, (1 << 23) + 128, P, 0, 4, None) == E_SHAPE   # 32-bit tile offsets
    assert mg(P, P, P, P, 0, 4, 1 << 23, None, 0, 4, None) == OK
    mp = lambda *a: _lib.status_of("mxfp4_gemm_debug_partials", *a)
    assert mp(P, P, P, P, 4, 4, 128, 0, 5, 0, 4, P, None) == E_SHAPE


def test_splitk_plan_and_validation(lib):
    wsb = _lib.splitk_workspace_bytes
    # LLaMA-2-70B w2 at M = 256: 2 x 64 tiles of 128 x 128 for 512 slots -> 4 splits of 56 stages
    assert wsb(256, 8192, 28672, 128, 128, 0) == 4 * 256 * 8192 * 4
    assert wsb(256, 8192, 28672, 128, 128, 3) == 3 * 256 * 8192 * 4
    assert wsb(256, 8192, 28672, 512, 128, 0) == 4 * 256 * 8192 * 4     # splits on 512-groups
    assert wsb(256, 8192, 28672, 128, 128, 1) == 0
    assert wsb(4096, 8192, 28672, 128, 128, 0) == 0                      # tiles fill the chip
    assert wsb(16, 8192, 28672, 128, 128, 0) == 0                        # few-token path
    assert wsb(300, 392, 1024, 128, 128, 100) == 8 * 300 * 392 * 4       # clamped to the 8 groups
    assert wsb(300, 392, 1024, 1024, 128, 100) == 8 * 300 * 392 * 4      # per-token A: W groups bound it
    assert wsb(300, 392, 1024, 256, 128, 100) == 8 * 300 * 392 * 4       # finer group 128
    assert wsb(300, 392, 1024, 256, 256, 100) == 4 * 300 * 392 * 4      # 2-stage groups
    assert lib.w4a4_gemm_splitk_workspace(4, 4, 96, 128, 128, 0) == -1
    assert lib.w4a4_gemm_splitk_workspace(4, 4, 256, 128, 128, -1) == -1
    assert lib.w4a4_gemm_splitk_workspace(4, 4, 256, 96, 128, 0) == -1
    sk = lambda *a: _lib.status_of("w4a4_gemm_splitk", *a)
    need = 4 * 256 * 8192 * 4
    assert sk(P, P, 128, P, P, 128, 256, 8192, 28672, 0, P, need - 4, P, 0, 8192, None) == E_SHAPE
    assert sk(P, P, 128, P, P, 128, 256, 8192, 28672, 0, None, need, P, 0, 8192, None) == E_NULL
    assert sk(P, P, 128, P, P, 128, 256, 8192, 28672, 0, P + 4, need, P, 0, 8192, None) == E_ALIGN
    assert sk(P, P, 128, P, P, 128, 256, 8192, 28672, -1, P, need, P, 0, 8192, None) == E_SHAPE
    assert sk(P, P, 128, P, P, 128, 256, 8192, 28672, 0, P, need, P, 3, 8192, None) == E_DTYPE
    assert sk(P, P, 96, P, P, 128, 256, 8192, 28672, 0, P, need, P, 0, 8192, None) == E_GROUP
    assert sk(P, P, 128, P, P, 128, 0, 8192, 28672, 0, None, 0, None, 0, 8192, None) == OK


def test_nvfp4_validation(lib):
    gs = lambda *a: _lib.status_of("nvfp4_global_scale", *a)
    assert gs(P, 4, 60, 60, P, None) == E_SHAPE          # K % 8
    assert gs(P, 4, 64, 68, P, None) == E_ALIGN
    assert gs(P, 4, 64, 64, None, None) == E_NULL
    assert gs(None, 4, 64, 64, P, None) == E_NULL
    assert gs(P + 8, 4, 64, 64, P, None) == E_ALIGN
    nq = lambda *a: _lib.status_of("nvfp4_quantize", *a)
    assert nq(P, 4, 128, 128, P, P, P, None) == E_SHAPE  # K % 256
    assert nq(P, 4, 256, 260, P, P, P, None) == E_ALIGN
    assert nq(P, 0, 256, 256, None, None, None, None) == OK
    assert nq(P, 4, 256, 256, None, P, P, None) == E_NULL
    assert nq(P, 4, 256, 256, P, P, P + 1, None) == E_ALIGN
    ng = lambda *a: _lib.status_of("nvfp4_gemm", *a)
    assert ng(P, P, P, P, P, P, 4, 4, 128, P, 0, 4, None) == E_SHAPE
    assert ng(P, P, P, P, P, P, 4, 4, 256, P, 2, 4, None) == E_DTYPE
    assert ng(P, P + 4, P, P, P, P, 4, 4, 256, P, 0, 4, None) == E_ALIGN   # scales 16-byte aligned
    assert ng(P, P, None, P, P, P, 4, 4, 256, P, 0, 4, None) == E_NULL
    assert ng(P, P, P, P, P, P, 0, 4, 256, None, 0, 4, None) == OK
    assert ng(P, P, P, P, P, P, 4, 4, (1 << 23) + 256, P, 0, 4, None) == E_SHAPE
    npart = lambda *a: _lib.status_of("nvfp4_gemm_debug_partials", *a)
    assert npart(P, P, P, P, 4, 4, 256, 0, 5, 0, 4, P, None) == E_SHAPE
    assert npart(P, P, P, P, 4, 4, 256, 0, 4, 0, 4, None, None) == E_NULL


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libw4a4.so"))
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load_library()


def test_storage_conversion_validation(lib):
    st = _lib.status_of
    assert st("w4a4_repack_int4", P, 4, 24, P, None, None) == E_SHAPE          # K % 16
    assert st("w4a4_repack_int4", P, -1, 32, P, None, None) == E_SHAPE
    assert st("w4a4_repack_int4", None, 4, 32, P, None, None) == E_NULL
    assert st("w4a4_repack_int4", P + 4, 4, 32, P, None, None) == E_ALIGN
    assert st("w4a4_repack_int4", P, 4, 32, P, P + 2, None) == E_ALIGN        # the count word
    assert st("w4a4_repack_int4", None, 0, 32, None, None, None) == OK          # empty, nothing counted
    assert st("w4a4_unpack_int4", P, 4, 40, P, None) == E_SHAPE
    assert st("w4a4_unpack_int4", P, 4, 32, None, None) == E_NULL
    assert st("w4a4_unpack_int4", P, 4, 32, P + 1, None) == E_ALIGN
    assert st("w4a4_scales_to_group_major", P, -1, 4, P, None) == E_SHAPE
    assert st("w4a4_scales_to_group_major", P, 65535 * 32 + 1, 4, P, None) == E_SHAPE
    assert st("w4a4_scales_to_group_major", P, 0, 4, None, None) == OK
    assert st("w4a4_scales_to_group_major", None, 3, 4, P, None) == E_NULL
    assert st("w4a4_scales_to_row_major", P + 2, 3, 4, P, None) == E_ALIGN
    assert st("mxfp4_scales_to_panels", P, 3, 48, P, None) == E_SHAPE          # K % 32
    assert st("mxfp4_scales_to_rows", None, 3, 64, P, None) == E_NULL
    assert st("nvfp4_scales_to_panels", P, 3, 128, P, None) == E_SHAPE         # K % 256
    assert st("nvfp4_scales_to_rows", P, 0, 256, None, None) == OK


def test_noalloc_splitk_validation(lib):
    """The no-allocation split-K entry point validates like w4a4_gemm_splitk and
    refuses a plan larger than its static buffer before any HIP call."""
    st = _lib.status_of
    M, N, K = 16, 32, 256
    assert lib.w4a4_gemm_splitk_noalloc_max_bytes() == 32 << 20
    assert st("w4a4_gemm_splitk_noalloc", P, P, 128, P, P, 128, M, N, 200, 0, P, 0, N, None) == E_SHAPE
    assert st("w4a4_gemm_splitk_noalloc", P, P, 96, P, P, 128, M, N, K, 0, P, 0, N, None) == E_GROUP
    assert st("w4a4_gemm_splitk_noalloc", P, P, 128, P, P, 128, M, N, K, -1, P, 0, N, None) == E_SHAPE
    assert st("w4a4_gemm_splitk_noalloc", P, P, 128, P, P, 128, M, N, K, 0, None, 0, N, None) == E_NULL
    assert st("w4a4_gemm_splitk_noalloc", P, P, 128, P, P, 128, 0, N, K, 0, None, 0, N, None) == OK
    # 8 splits of 512 x 8192 fp32 = 128 MiB > 32 MiB: W4A4_E_SCRATCH
    assert st("w4a4_gemm_splitk_noalloc", P, P, 128, P, P, 128, 512, 8192, 4096, 8, P, 0, 8192, None) == 7
    assert lib.w4a4_status_str(7) != b"unknown status"


def test_probe_validation(lib):
    st = _lib.status_of
    assert lib.w4a4_probe_sink_bytes() >= 4 * 2048 * 256
    assert lib.w4a4_probe_mfma_ops(0, 10) == 2 * 32 * 32 * 32 * 4 * 10 * 4 * 2048
    assert lib.w4a4_probe_mfma_ops(2, 10) == 2 * lib.w4a4_probe_mfma_ops(0, 10)
    assert lib.w4a4_probe_mfma_ops(9, 10) == -1
    assert st("w4a4_probe_mfma", 6, 10, P, None) == E_SHAPE
    assert lib.w4a4_probe_mfma_ops(5, 10) == 2 * 64 * 64 * 10 * 4 * 2048   # 64 fmas per lane per iteration
    assert st("w4a4_probe_mfma", 0, 0, P, None) == E_SHAPE
    assert st("w4a4_probe_mfma", 0, 10, None, None) == E_NULL
    assert st("w4a4_probe_hbm_read", P, 24, P, None) == E_SHAPE
    assert st("w4a4_probe_hbm_read", P + 8, 32, P, None) == E_ALIGN
    assert st("w4a4_probe_hbm_copy", P, 32, None, None) == E_NULL


def test_fused_linear_validation(lib):
    st = _lib.status_of
    sup = lib.w4a4_linear_fused_supported
    assert sup(1, 28672, 8192, 128, 128) == 1 and sup(8, 28672, 8192, 128, 128) == 1
    # the fused path's 16-column tiles (4 accumulators per lane to sum across
    # waves): M = 9 fits 64 KiB at K = 8192, M = 10 does not; M = 2 at K = 28672,
    # M = 3 not
    assert sup(9, 28672, 8192, 128, 128) == 1 and sup(10, 28672, 8192, 128, 128) == 0
    assert sup(2, 8192, 28672, 128, 128) == 1 and sup(3, 8192, 28672, 128, 128) == 0
    # groups of 64 take the 32-column tiles (16 accumulators per lane)
    assert sup(2, 8192, 8192, 64, 64) == 1 and sup(4, 8192, 28672, 64, 64) == 0
    assert sup(33, 64, 256, 128, 128) == 0 and sup(4, 64, 1024, 1024, 128) == 0   # per-token A: not fused
    assert sup(4, 64, 1024, 96, 128) == 0 and sup(0, 64, 256, 128, 128) == 0
    f = "w4a4_linear_fused"
    assert st(f, P, 2, 200, 200, 128, P, P, 128, 64, P, 0, 64, None) == E_SHAPE     # K % 128
    assert st(f, P, 2, 256, 248, 128, P, P, 128, 64, P, 0, 64, None) == E_SHAPE     # ldx < K
    assert st(f, P, 2, 256, 260, 128, P, P, 128, 64, P, 0, 64, None) == E_ALIGN     # ldx % 8
    assert st(f, P, 2, 256, 256, 96, P, P, 128, 64, P, 0, 64, None) == E_GROUP
    assert st(f, P, 40, 256, 256, 128, P, P, 128, 64, P, 0, 64, None) == E_SHAPE    # M > 32
    assert st(f, P, 2, 256, 256, 128, P, P, 128, 64, P, 0, 32, None) == E_SHAPE     # ldy < N
    assert st(f, None, 2, 256, 256, 128, P, P, 128, 64, P, 0, 64, None) == E_NULL
    assert st(f, P + 8, 2, 256, 256, 128, P, P, 128, 64, P, 0, 64, None) == E_ALIGN
    assert st(f, None, 0, 256, 256, 128, None, None, 128, 64, None, 0, 64, None) == OK   # empty


def test_fused_policy_choices(lib):
    """w4a4_linear's own choice of the fused launch (host logic): the measured
    decode crossovers (LLaMA-2-70B w1/w3 fused up to M = 3; LLaMA-2-7B up to
    M = 5), never past the kernel's LDS limit, never for empty shapes."""
    from w4a4_quantized_gemm_quantize_amd import ops
    picks = lambda N, K: [M for M in range(1, 33) if ops.use_fused(M, N, K, 128, 128)]
    assert picks(28672, 8192) == [1, 2, 3]          # LLaMA-2-70B w1 / w3
    assert picks(8192, 28672) == [1, 2]             # w2: the LDS copy of X fits M <= 2
    assert picks(11008, 4096) == [1, 2, 3, 4, 5]    # LLaMA-2-7B w1 / w3
    assert picks(4096, 11008) == [1, 2, 3, 4, 5]    # LLaMA-2-7B w2
    for M, N, K in ((0, 64, 256), (1, 0, 256)):
        assert not ops.use_fused(M, N, K, 128, 128)
    for M in range(1, 33):                          # the policy never asks for an unsupported launch
        for N, K in ((28672, 8192), (8192, 28672), (11008, 4096), (64, 1024)):
            if ops.use_fused(M, N, K, 128, 128):
                assert lib.w4a4_linear_fused_supported(M, N, K, 128, 128) == 1
