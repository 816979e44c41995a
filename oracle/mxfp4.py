"""MXFP4 quantization and the block-scaled FP4 GEMM (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name the format only: "the open-standard MXFP4" (FP4 RL post-training
abstract on the "Depth Registers Unlock W4A4 on SwiGLU" page), "microscaled FP4
formats" (ReQAT abstract, "Hardware-Aware FP4 FlashAttention-4" page) and MXFP4
weights with a per-block error bound (Multi-Scale Dequant abstract, APEX4 page).
The open standard is the OCP Microscaling Formats (MX) v1.0 specification; the
readings taken from it here:

* blocks of 32 consecutive K elements share one E8M0 scale 2^E (byte E + 127);
* elements are FP4 E2M1 (1 sign, 2 exponent bits with bias 1, 1 mantissa bit):
  magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}, code = sign<<3 | index;
* ``E = floor(log2(max|x|)) - 2`` (2 = exponent of the largest E2M1 value);
  an all-zero block takes E = -127 (byte 0);
* ``v = x / 2^E`` (exact), rounded to the nearest E2M1 magnitude with ties to the
  even code (mantissa bit 0), magnitudes above 6 saturating to 6; the sign bit
  of x is kept, also when the magnitude rounds to 0;
* packing as for INT4: two codes per byte, even k in the low nibble.

GEMM: ``Y = sum_b 2^(Ea_b + Ew_b) * sum_{k in b} va*vw``. With ``I_b =
sum_{k in b} (2va)(2vw)`` (an exact integer), ``Y = sum_b I_b 2^(Ea+Ew-2)``.
"""
from __future__ import annotations

import numpy as np

MX_BLOCK = 32
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_MAX = 6.0
E2M1_EMAX = 2          # exponent of the largest normal E2M1 value (6 = 1.5 * 2^2)
E8M0_BIAS = 127


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """4-bit E2M1 codes (0..15) -> float64 values."""
    c = np.asarray(codes).astype(np.int64)
    mag = E2M1_VALUES[c & 7]
    return np.where(c & 8, -mag, mag)


def _round_to_e2m1_index(m: np.ndarray) -> np.ndarray:
    """Index into E2M1_VALUES of the RNE rounding of non-negative ``m`` (saturating)."""
    m = np.minimum(m, E2M1_MAX)                          # saturate
    hi = np.searchsorted(E2M1_VALUES, m, side="left")    # first grid point >= m
    hi = np.minimum(hi, len(E2M1_VALUES) - 1)
    lo = np.where(E2M1_VALUES[hi] == m, hi, np.maximum(hi - 1, 0))
    d_lo = m - E2M1_VALUES[lo]
    d_hi = E2M1_VALUES[hi] - m
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    return np.where(pick_hi, hi, lo).astype(np.int64)


def _mx_rule(xf: np.ndarray):
    """The OCP MX block rule above on finite float64 values [R, K] (K % 32 == 0).

    Returns ``(codes, e8m0)``: codes uint8 [R, K] holding 0..15, scale bytes
    uint8 [R, K/32].
    """
    R, K = xf.shape
    xb = xf.reshape(R, K // MX_BLOCK, MX_BLOCK)
    a = np.abs(xb).max(axis=2)
    _, e = np.frexp(a)                                   # a = f * 2^e, f in [0.5, 1)
    E = np.where(a > 0, (e - 1) - E2M1_EMAX, -E8M0_BIAS)  # floor(log2 a) - 2
    E = np.clip(E, -E8M0_BIAS, E8M0_BIAS).astype(np.int64)
    v = np.ldexp(xb, -E[:, :, None])                     # exact scaling by 2^-E
    idx = _round_to_e2m1_index(np.abs(v))
    sign = np.signbit(xb).astype(np.int64)
    codes = (sign << 3) | idx
    return codes.reshape(R, K).astype(np.uint8), (E + E8M0_BIAS).astype(np.uint8)


def mxfp4_quantize(x: np.ndarray):
    """MXFP4-quantize each row in blocks of 32 along K.

    Returns ``(codes, e8m0)``: codes uint8 [R, K] holding 0..15, scale bytes
    uint8 [R, K/32].
    """
    x = np.asarray(x)
    if x.dtype != np.float16 or x.ndim != 2:
        raise TypeError("x must be a 2-D float16 array")
    R, K = x.shape
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    xf = x.astype(np.float64)                            # exact
    if not np.isfinite(xf).all():
        raise ValueError("NaN/Inf inputs are outside the quantizer's contract")
    return _mx_rule(xf)


def mxfp4_quantize_residual(x: np.ndarray):
    """Two-pass MXFP4 with the residual pass appended along K.

    Multi-Scale Dequant abstract (APEX4 page): the high-precision activation is
    decomposed into several low-precision components, each multiplied with the
    quantized weights by the native GEMM; for MXFP4 two passes. ARCQuant
    abstract (same page): the quantized residual is appended to the activation
    as extra channels of the reduction dimension, so one standard GEMM computes
    both terms. The pages give only these abstracts; reading taken here (the
    plainest): the second pass is the same MX rule applied to the exact residual
    ``R = x - deq(Q(x))``, with its own per-block scale. ``R`` is exact in
    float64 (and in binary32: it needs at most 16 significant bits).

    Returns ``(codes, e8m0)`` of the augmented activation: codes uint8
    [R, 2K] = [Q(x) | Q(R)], scale bytes uint8 [R, 2K/32].
    """
    c1, e1 = mxfp4_quantize(x)
    r = np.asarray(x).astype(np.float64) - mxfp4_dequantize(c1, e1)
    c2, e2 = _mx_rule(r)
    return np.concatenate([c1, c2], axis=1), np.concatenate([e1, e2], axis=1)


def mxfp4_append_copy(codes: np.ndarray, e8m0: np.ndarray):
    """The weight side of the appended-residual GEMM: each row's codes and
    scales twice along K, so that [Q(x) | Q(R)] @ [Q(w) | Q(w)]^T =
    Q(x) Q(w)^T + Q(R) Q(w)^T."""
    return np.concatenate([codes, codes], axis=1), np.concatenate([e8m0, e8m0], axis=1)


def mxfp4_dequantize(codes: np.ndarray, e8m0: np.ndarray) -> np.ndarray:
    """x_hat = v * 2^E in float64 (exact)."""
    v = e2m1_decode(codes)
    E = np.repeat(e8m0.astype(np.int64) - E8M0_BIAS, MX_BLOCK, axis=1)
    return np.ldexp(v, E)


def mxfp4_block_partials(ca: np.ndarray, cw: np.ndarray):
    """Yield ``(b, I_b)`` with ``I_b = (2 va_b) @ (2 vw_b)^T`` as int64.

    2*v is an integer in [-12, 12]; the float64 library matmul of such integers
    is exact.
    """
    R, K = ca.shape
    if cw.shape[1] != K or K % MX_BLOCK:
        raise ValueError("K mismatch or not a multiple of 32")
    for b in range(K // MX_BLOCK):
        A = 2.0 * e2m1_decode(ca[:, b * MX_BLOCK:(b + 1) * MX_BLOCK])
        W = 2.0 * e2m1_decode(cw[:, b * MX_BLOCK:(b + 1) * MX_BLOCK])
        yield b, (A @ W.T).astype(np.int64)


def mxfp4_gemm(ca: np.ndarray, ea: np.ndarray, cw: np.ndarray, ew: np.ndarray):
    """Block-scaled FP4 GEMM; returns ``(Y, T)`` in float64.

    ``Y[m,n] = sum_b I_b[m,n] * 2^(Ea[m,b] + Ew[n,b] - 2)`` in block order; each
    term is exact, ``T`` is the sum of their absolute values.
    """
    M, K = ca.shape
    N = cw.shape[0]
    if ea.shape != (M, K // MX_BLOCK) or ew.shape != (N, K // MX_BLOCK):
        raise ValueError("scale shapes do not match")
    Ea = ea.astype(np.int64) - E8M0_BIAS
    Ew = ew.astype(np.int64) - E8M0_BIAS
    Y = np.zeros((M, N), dtype=np.float64)
    T = np.zeros((M, N), dtype=np.float64)
    for b, I in mxfp4_block_partials(ca, cw):
        term = np.ldexp(I.astype(np.float64), Ea[:, b][:, None] + Ew[:, b][None, :] - 2)
        Y += term
        T += np.abs(term)
    return Y, T
