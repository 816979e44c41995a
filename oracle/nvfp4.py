"""NVFP4 quantization and the two-level-scaled FP4 GEMM (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix: NVFP4 is a fine-grained FP4 format that a unified,
standard GEMM consumes (ARCQuant abstract, APEX4 page); its scaling is per
block of 16 elements, which keeps a single outlier from widening the scale of
more than its own 16 neighbours, and a checkpoint also carries a global scale
per module, calibrated, which must agree across modules that one GEMM fuses
(Minima abstract, "Daily Papers" page). The pages give no element type, scale
type, formula or rounding. The readings taken here are those of the format's
public definition and the plainest arithmetic around it:

* elements are FP4 E2M1 (the type MXFP4 also uses): magnitudes {0, 0.5, 1,
  1.5, 2, 3, 4, 6}, code = sign << 3 | index, two codes per byte with the even
  k in the low nibble;
* each block of 16 consecutive K elements of a row has a scale s_b stored as
  one byte of OCP FP8 E4M3 (E4M3FN: bias 7, subnormals, no infinities, 448 the
  largest finite value, S.1111.111 the only NaN);
* the tensor has one binary32 scale s_g > 0 (the global scale) multiplying
  every block scale: x_hat = v * s_b * s_g;
* the global scale is supplied by the caller (a calibrated value), or taken
  from the tensor's own absmax as ``s_g = fl32(amax / 2688)``, 2688 = 6 * 448,
  so that the block holding the absmax gets the largest E4M3 scale;
* per block with absmax a (exact): ``d = fl32(6 s_g)``; a = 0 gives s_b = 0;
  otherwise ``r = min(fl32(a / d), 448)`` (d = 0 makes r = +inf, saturated) and
  s_b = E4M3 rounding of r to nearest, ties to the even code;
* the block's encode factor is ``e = fl32(1 / fl32(s_b s_g))`` (e = 0 when that
  product is 0) and each element's code is the E2M1 rounding of
  ``t = fl32(x e)`` to nearest, ties to the even code, magnitudes above 6
  saturating to 6, the sign bit that of x (also when the magnitude rounds
  to 0). Dividing by the scale is read as multiplying by its binary32
  reciprocal, one division per block; every binary32 step is correctly
  rounded -- the precision the GPU kernel takes the same decisions in.

GEMM: ``Y = X W^T``, ``Y[m, n] = g_a g_w sum_b s_a[m, b] s_w[n, b]
sum_{k in b} va vw`` with ``I_b = sum_{k in b} (2 va)(2 vw)`` an exact
integer (|I_b| <= 16 * 144), i.e. ``Y = g_a g_w sum_b I_b s_a s_w / 4``.
"""
from __future__ import annotations

import numpy as np

from .mxfp4 import E2M1_MAX, _round_to_e2m1_index, e2m1_decode

NV_BLOCK = 16
E4M3_MAX = 448.0
E4M3_BIAS = 7
E4M3_NAN = 0x7F
E4M3_MIN_NORMAL_EXP = -6          # smallest normal value 2^-6
E4M3_MANT_BITS = 3
GLOBAL_DIVISOR = np.float32(E2M1_MAX * E4M3_MAX)   # 2688


def e4m3_decode(b: np.ndarray) -> np.ndarray:
    """FP8 E4M3 (E4M3FN) bytes -> float64 values (NaN for S.1111.111)."""
    b = np.asarray(b).astype(np.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e == 0,
                   np.ldexp(m.astype(np.float64) / 8.0, E4M3_MIN_NORMAL_EXP),
                   np.ldexp(1.0 + m.astype(np.float64) / 8.0, e - E4M3_BIAS))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def e4m3_round(r: np.ndarray) -> np.ndarray:
    """Byte of the E4M3 value nearest to each non-negative ``r`` <= 448 (finite),
    ties to the even code.

    The representable values of binade [2^E, 2^(E+1)) (E >= -6) are spaced
    2^(E-3) apart; below 2^-6 (subnormals) the spacing is 2^-9. ``r / spacing``
    is exact in float64; rounding it half-to-even picks the value, and an
    even multiple of the spacing is a code with mantissa bit 0.
    """
    r = np.asarray(r, dtype=np.float64)
    if np.any(~np.isfinite(r)) or np.any(r < 0) or np.any(r > E4M3_MAX):
        raise ValueError("e4m3_round takes finite values in [0, 448]")
    _, ex = np.frexp(r)                               # r = f 2^ex, f in [0.5, 1)
    E = np.maximum(ex - 1, E4M3_MIN_NORMAL_EXP)       # binade of r (subnormals share -6)
    spacing_exp = E - E4M3_MANT_BITS
    n = np.rint(np.ldexp(r, -spacing_exp))            # half to even
    v = np.ldexp(n, spacing_exp)                      # the rounded value
    # encode v: subnormal (v < 2^-6) has exponent field 0, mantissa n
    _, ev = np.frexp(v)
    Ev = ev - 1
    normal = v >= 2.0 ** E4M3_MIN_NORMAL_EXP
    efield = np.where(normal, Ev + E4M3_BIAS, 0)
    mfield = np.where(normal, np.ldexp(v, -(Ev - E4M3_MANT_BITS)) - 8, np.ldexp(v, 9))
    return (efield * 8 + mfield).astype(np.uint8)


def nvfp4_global_scale(x: np.ndarray) -> np.float32:
    """``fl32(amax / 2688)`` of a float16 tensor (0 for an all-zero tensor)."""
    x = np.asarray(x)
    if x.dtype != np.float16:
        raise TypeError("x must be float16")
    xf = x.astype(np.float32)
    if not np.isfinite(xf).all():
        raise ValueError("NaN/Inf inputs are outside the quantizer's contract")
    amax = np.float32(np.abs(xf).max()) if xf.size else np.float32(0)
    return np.float32(amax / GLOBAL_DIVISOR)


def nvfp4_quantize(x: np.ndarray, global_scale):
    """NVFP4-quantize each row in blocks of 16 along K with the global scale.

    Returns ``(codes, sbytes)``: codes uint8 [R, K] holding 0..15, E4M3 scale
    bytes uint8 [R, K/16]. Follows the steps of the module docstring, in order.
    """
    x = np.asarray(x)
    if x.dtype != np.float16 or x.ndim != 2:
        raise TypeError("x must be a 2-D float16 array")
    R, K = x.shape
    if K % NV_BLOCK:
        raise ValueError("K must be a multiple of 16")
    sg = np.float32(global_scale)
    if not np.isfinite(sg) or sg < 0:
        raise ValueError("the global scale must be finite and >= 0")
    xf = x.astype(np.float32)                           # exact
    if not np.isfinite(xf).all():
        raise ValueError("NaN/Inf inputs are outside the quantizer's contract")
    xb = xf.reshape(R, K // NV_BLOCK, NV_BLOCK)
    a = np.abs(xb).max(axis=2)                           # exact
    d = np.float32(np.float32(6.0) * sg)                # binary32 product
    with np.errstate(divide="ignore", invalid="ignore"):
        r = (a / d).astype(np.float32)                   # binary32 division
    r = np.where(a == 0, np.float32(0), np.minimum(r, np.float32(E4M3_MAX)))
    sbytes = e4m3_round(r)
    sb = e4m3_decode(sbytes).astype(np.float32)         # exact
    S = (sb * sg).astype(np.float32)                     # binary32 product
    with np.errstate(divide="ignore"):
        e = np.where(S == 0, np.float32(0), (np.float32(1.0) / S)).astype(np.float32)
    t = (xb * e[:, :, None]).astype(np.float32)          # binary32 product, sign of x
    idx = _round_to_e2m1_index(np.abs(t.astype(np.float64)))
    sign = np.signbit(xb).astype(np.int64)
    codes = (sign << 3) | idx
    return codes.reshape(R, K).astype(np.uint8), sbytes


def nvfp4_dequantize(codes: np.ndarray, sbytes: np.ndarray, global_scale) -> np.ndarray:
    """x_hat = v * s_b * s_g in float64 (exact: 2 + 4 + 24 significant bits)."""
    v = e2m1_decode(codes)
    sb = np.repeat(e4m3_decode(sbytes), NV_BLOCK, axis=1)
    return v * sb * np.float64(np.float32(global_scale))


def nvfp4_block_partials(ca: np.ndarray, cw: np.ndarray):
    """Yield ``(b, I_b)`` with ``I_b = (2 va_b) @ (2 vw_b)^T`` as int64 (exact)."""
    R, K = ca.shape
    if cw.shape[1] != K or K % NV_BLOCK:
        raise ValueError("K mismatch or not a multiple of 16")
    for b in range(K // NV_BLOCK):
        A = 2.0 * e2m1_decode(ca[:, b * NV_BLOCK:(b + 1) * NV_BLOCK])
        W = 2.0 * e2m1_decode(cw[:, b * NV_BLOCK:(b + 1) * NV_BLOCK])
        yield b, (A @ W.T).astype(np.int64)


def nvfp4_gemm(ca, sa, ga, cw, sw, gw):
    """Two-level-scaled FP4 GEMM; returns ``(Y, T)`` in float64.

    ``Y[m, n] = g_a g_w sum_b I_b[m, n] s_a[m, b] s_w[n, b] / 4`` in block
    order; ``T`` is the same sum of absolute values (it scales the parity
    tolerance).
    """
    M, K = ca.shape
    N = cw.shape[0]
    if sa.shape != (M, K // NV_BLOCK) or sw.shape != (N, K // NV_BLOCK):
        raise ValueError("scale shapes do not match the codes")
    SA = e4m3_decode(sa)
    SW = e4m3_decode(sw)
    G = np.float64(np.float32(ga)) * np.float64(np.float32(gw))
    Y = np.zeros((M, N))
    T = np.zeros((M, N))
    for b, I in nvfp4_block_partials(ca, cw):
        term = I * np.outer(SA[:, b], SW[:, b]) * 0.25
        Y += term
        T += np.abs(term)
    return Y * G, T * abs(G)
