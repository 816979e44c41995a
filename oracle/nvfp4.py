"""NVFP4 quantization and the two-level-scaled FP4 GEMM (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring). The arithmetic is the
C++ of ``orc.cpp`` (``e4m3_round``, ``nvfp4_global_scale``,
``nvfp4_quantize``, ``nvfp4_gemm``); this module passes numpy arrays to it.

What the pages fix: NVFP4 is a fine-grained FP4 format that a unified,
standard GEMM consumes (ARCQuant abstract, APEX4 page); its scaling is per
block of 16 elements, which keeps a single outlier from widening the scale of
more than its own 16 neighbours, and a checkpoint also carries a global scale
per module, calibrated, which must agree across modules that one GEMM fuses
(Minima abstract, "Daily Papers" page). The pages give no element type, scale
type, formula or rounding. The readings taken are those of the format's
public definition and the plainest arithmetic around it:

* elements are FP4 E2M1 (the type MXFP4 also uses), code = sign << 3 | index;
* each block of 16 consecutive K elements of a row has a scale s_b stored as
  one byte of OCP FP8 E4M3 (E4M3FN: bias 7, subnormals, no infinities, 448 the
  largest finite value, S.1111.111 the only NaN);
* the tensor has one binary32 scale s_g >= 0 (the global scale) multiplying
  every block scale: x_hat = v * s_b * s_g; by default ``s_g = fl32(amax /
  2688)``, 2688 = 6 * 448, so the block holding the absmax gets the largest
  E4M3 scale;
* per block with absmax a: ``d = fl32(6 s_g)``; a = 0 gives s_b = 0; otherwise
  ``r = min(fl32(a / d), 448)`` and s_b = E4M3 rounding of r to nearest, ties
  to the even code;
* the encode factor is ``e = fl32(1 / fl32(s_b s_g))`` (0 when that product is
  0) and each element's code is the E2M1 rounding of ``t = fl32(x e)`` (ties
  to even, saturating at 6, the sign bit that of x). Dividing by the scale is
  read as multiplying by its binary32 reciprocal, one division per block.

GEMM: ``Y[m, n] = g_a g_w sum_b s_a[m, b] s_w[n, b] sum_{k in b} va vw``, with
``I_b = sum_{k in b} (2 va)(2 vw)`` an exact integer: ``Y = g_a g_w sum_b I_b
s_a s_w / 4``.
"""
from __future__ import annotations

import numpy as np

from . import _native as nat
from .mxfp4 import fp4_block_partials

NV_BLOCK = 16
E4M3_MAX = 448.0


def e4m3_decode(b: np.ndarray) -> np.ndarray:
    """FP8 E4M3 (E4M3FN) bytes -> float64 values (NaN for S.1111.111)."""
    table = np.array([nat.lib().orc_e4m3_value(i) for i in range(256)], dtype=np.float64)
    return table[np.asarray(b).astype(np.int64) & 255]


def e4m3_round(r: np.ndarray) -> np.ndarray:
    """Byte of the E4M3 value nearest to each non-negative ``r`` <= 448 (finite),
    ties to the even code."""
    r = np.asarray(r, dtype=np.float64)
    if np.any(~np.isfinite(r)) or np.any(r < 0) or np.any(r > E4M3_MAX):
        raise ValueError("e4m3_round takes finite values in [0, 448]")
    f = nat.lib().orc_e4m3_round
    return np.array([f(float(v)) for v in r.reshape(-1)], dtype=np.uint8).reshape(r.shape)


def nvfp4_global_scale(x: np.ndarray) -> np.float32:
    """``fl32(amax / 2688)`` of a float16 tensor (0 for an empty or all-zero tensor)."""
    x = np.asarray(x)
    if x.dtype != np.float16:
        raise TypeError("x must be float16")
    xb = np.ascontiguousarray(x).view(np.uint16).reshape(-1)
    out = np.zeros(1, dtype=np.float32)
    nat.check(nat.lib().orc_nvfp4_global_scale(nat.ptr(xb), xb.size, nat.ptr(out)))
    return np.float32(out[0])


def nvfp4_quantize(x: np.ndarray, global_scale):
    """NVFP4-quantize each row in blocks of 16 along K with the global scale.

    Returns ``(codes, sbytes)``: codes uint8 [R, K] holding 0..15, E4M3 scale
    bytes uint8 [R, K/16].
    """
    x = np.asarray(x)
    if x.dtype != np.float16 or x.ndim != 2:
        raise TypeError("x must be a 2-D float16 array")
    xb = np.ascontiguousarray(x).view(np.uint16)
    R, K = xb.shape
    if K % NV_BLOCK:
        raise ValueError("K must be a multiple of 16")
    codes = np.empty((R, K), dtype=np.uint8)
    sbytes = np.empty((R, K // NV_BLOCK), dtype=np.uint8)
    nat.check(nat.lib().orc_nvfp4_quantize(nat.ptr(xb), R, K, float(np.float32(global_scale)),
                                           nat.ptr(codes), nat.ptr(sbytes), nat.threads))
    return codes, sbytes


def nvfp4_dequantize(codes: np.ndarray, sbytes: np.ndarray, global_scale) -> np.ndarray:
    """x_hat = v * s_b * s_g in float64 (exact: 2 + 4 + 24 significant bits)."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    s = np.ascontiguousarray(sbytes, dtype=np.uint8)
    R, K = c.shape
    if K % NV_BLOCK or s.shape != (R, K // NV_BLOCK):
        raise ValueError("scale shape does not match the codes")
    out = np.empty((R, K), dtype=np.float64)
    nat.lib().orc_nvfp4_dequantize(nat.ptr(c), nat.ptr(s), float(np.float32(global_scale)), R, K, nat.ptr(out))
    return out


def nvfp4_block_partials(ca: np.ndarray, cw: np.ndarray):
    """Yield ``(b, I_b)`` with ``I_b = (2 va_b) @ (2 vw_b)^T`` as int64 (exact)."""
    P = fp4_block_partials(ca, cw, NV_BLOCK)
    for b in range(P.shape[0]):
        yield b, P[b].astype(np.int64)


def nvfp4_gemm(ca, sa, ga, cw, sw, gw):
    """Two-level-scaled FP4 GEMM; returns ``(Y, T)`` in float64.

    ``Y[m, n] = g_a g_w sum_b I_b[m, n] s_a[m, b] s_w[n, b] / 4`` in block
    order; ``T`` is the same sum of absolute values (it scales the parity
    tolerance).
    """
    a = np.ascontiguousarray(ca, dtype=np.uint8)
    w = np.ascontiguousarray(cw, dtype=np.uint8)
    M, K = a.shape
    N = w.shape[0]
    s_a = np.ascontiguousarray(sa, dtype=np.uint8)
    s_w = np.ascontiguousarray(sw, dtype=np.uint8)
    if w.shape[1] != K or K % NV_BLOCK or s_a.shape != (M, K // NV_BLOCK) or s_w.shape != (N, K // NV_BLOCK):
        raise ValueError("scale shapes do not match the codes")
    Y = np.empty((M, N), dtype=np.float64)
    T = np.empty((M, N), dtype=np.float64)
    nat.check(nat.lib().orc_nvfp4_gemm(nat.ptr(a), nat.ptr(s_a), float(np.float32(ga)), nat.ptr(w), nat.ptr(s_w),
                                       float(np.float32(gw)), M, N, K, nat.ptr(Y), nat.ptr(T), nat.threads))
    return Y, T
