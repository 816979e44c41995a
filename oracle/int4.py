"""INT4 symmetric group quantization and the W4A4 group-dequantized GEMM (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring). The arithmetic is the
C++ of ``orc.cpp`` (``int4_quantize``, ``w4a4_block_partials``,
``w4a4_gemm``); this module passes numpy arrays to it.

What the pages fix ("APEX4: Efficient Pure W4A4 LLM Inference via Intra-SM
Compute Rebalancing", abstract): 4-bit weights AND 4-bit activations, groups of
128 along the reduction axis ("W4A4-g128"), a pure INT4 matrix product whose
per-group results are then dequantized by the vector units, and a
mixed-granularity mode in which the activation group size differs from the
weight one. They give no quantization formula, rounding mode, scale type or
layout. The readings taken:

* symmetric, no zero point; per row and per group of ``g`` consecutive K
  elements: ``a = max|x|``, ``s = fl32(a / 7)``, ``q = clamp(rne(fl32(x / s)),
  -8, 7)``; an all-zero group has ``s = 0`` and codes 0;
* scales are IEEE binary32; divisions are correctly rounded binary32 (the
  precision the kernel makes the integer decision in); ties round to even;
* codes are integers (two's complement); how they are stored is
  :mod:`oracle.layout`'s business, not this module's;
* the GEMM is ``Y = X W^T`` (a linear layer), A = activations [M, K] and
  W = weights [N, K]; with ``g = min(g_a, g_w)`` (nested groups) the per-block
  integer partial is ``P_b[m, n] = sum_{k in block b} qa[m,k] qw[n,k]`` and
  ``Y[m, n] = sum_b s_a[m, b g/g_a] s_w[n, b g/g_w] P_b[m, n]`` -- the
  dequantization folded into the accumulation, block by block;
* ``T[m, n] = sum_b |s_a s_w P_b|`` is returned beside ``Y``: it scales the
  tolerance ``|Y_gpu - Y| <= 1e-5 T + 1e-6`` used by the parity tests.
"""
from __future__ import annotations

import numpy as np

from . import _native as nat


def _f16_bits(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype != np.float16 or x.ndim != 2:
        raise TypeError("x must be a 2-D float16 array")
    return np.ascontiguousarray(x).view(np.uint16)


def int4_quantize(x: np.ndarray, group: int):
    """Symmetric INT4 quantization of each row in groups of ``group`` along K.

    Returns ``(codes, scales)``: codes int8 [R, K] in [-8, 7], scales float32
    [R, K/group] (row-major).
    """
    xb = _f16_bits(x)
    R, K = xb.shape
    if group <= 0 or K % group:
        raise ValueError(f"group {group} must divide K={K}")
    codes = np.empty((R, K), dtype=np.int8)
    scales = np.empty((R, K // group), dtype=np.float32)
    nat.check(nat.lib().orc_int4_quantize(nat.ptr(xb), R, K, group, nat.ptr(codes), nat.ptr(scales),
                                          nat.threads))
    return codes, scales


def int4_dequantize(codes: np.ndarray, scales: np.ndarray, group: int) -> np.ndarray:
    """x_hat = q * s in float64 (exact: 4-bit times 24-bit significands)."""
    q = np.ascontiguousarray(codes, dtype=np.int8)
    s = np.ascontiguousarray(scales, dtype=np.float32)
    R, K = q.shape
    if group <= 0 or K % group or s.shape != (R, K // group):
        raise ValueError("scale shape does not match the group size")
    out = np.empty((R, K), dtype=np.float64)
    nat.lib().orc_int4_dequantize(nat.ptr(q), nat.ptr(s), R, K, group, nat.ptr(out))
    return out


def w4a4_block_partials(qa: np.ndarray, qw: np.ndarray, g: int):
    """Yield ``(b, P_b)`` with ``P_b[m, n] = sum_{k in block b} qa[m,k] qw[n,k]``
    (int64 sums in the oracle, int32 results)."""
    a = np.ascontiguousarray(qa, dtype=np.int8)
    w = np.ascontiguousarray(qw, dtype=np.int8)
    M, K = a.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("K mismatch")
    if g <= 0 or K % g:
        raise ValueError(f"group {g} must divide K={K}")
    P = np.empty((K // g, M, N), dtype=np.int32)
    nat.check(nat.lib().orc_w4a4_block_partials(nat.ptr(a), nat.ptr(w), M, N, K, g, nat.ptr(P), nat.threads))
    for b in range(K // g):
        yield b, P[b].astype(np.int64)


def w4a4_gemm(qa: np.ndarray, sa: np.ndarray, g_a: int,
              qw: np.ndarray, sw: np.ndarray, g_w: int):
    """Group-dequantized INT4 GEMM; returns ``(Y, T)`` in float64.

    ``Y[m,n] = sum_b s_a[m, b g/g_a] * s_w[n, b g/g_w] * P_b[m,n]`` summed in
    block order; ``T`` is the same sum of absolute values.
    """
    a = np.ascontiguousarray(qa, dtype=np.int8)
    w = np.ascontiguousarray(qw, dtype=np.int8)
    M, K = a.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("K mismatch")
    if g_a <= 0 or g_w <= 0 or K % g_a or K % g_w:
        raise ValueError("groups must divide K")
    if max(g_a, g_w) % min(g_a, g_w):
        raise ValueError("activation and weight groups must nest")
    sa32 = np.ascontiguousarray(sa, dtype=np.float32)
    sw32 = np.ascontiguousarray(sw, dtype=np.float32)
    if sa32.shape != (M, K // g_a) or sw32.shape != (N, K // g_w):
        raise ValueError("scale shapes do not match the groups")
    Y = np.empty((M, N), dtype=np.float64)
    T = np.empty((M, N), dtype=np.float64)
    nat.check(nat.lib().orc_w4a4_gemm(nat.ptr(a), nat.ptr(sa32), g_a, nat.ptr(w), nat.ptr(sw32), g_w,
                                      M, N, K, nat.ptr(Y), nat.ptr(T), nat.threads))
    return Y, T


def w4a4_gemm_rows(qa: np.ndarray, sa: np.ndarray, g_a: int,
                   qw: np.ndarray, sw: np.ndarray, g_w: int, rows) -> tuple:
    """:func:`w4a4_gemm` restricted to the listed output rows (same arithmetic)."""
    rows = np.asarray(rows, dtype=np.int64)
    return w4a4_gemm(qa[rows], sa[rows], g_a, qw, sw, g_w)
