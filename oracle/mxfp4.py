"""MXFP4 quantization and the block-scaled FP4 GEMM (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring). The arithmetic is the
C++ of ``orc.cpp`` (``mx_block``, ``mxfp4_quantize``,
``mxfp4_quantize_residual``, ``fp4_block_partials``, ``mxfp4_gemm``); this
module passes numpy arrays to it.

The pages name the format only: "the open-standard MXFP4" (FP4 RL post-training
abstract on the "Depth Registers Unlock W4A4 on SwiGLU" page), "microscaled FP4
formats" (ReQAT abstract, "Hardware-Aware FP4 FlashAttention-4" page) and MXFP4
weights with a per-block error bound (Multi-Scale Dequant abstract, APEX4 page).
The open standard is the OCP Microscaling Formats (MX) v1.0 specification; the
readings taken from it:

* blocks of 32 consecutive K elements share one E8M0 scale 2^E (byte E + 127);
* elements are FP4 E2M1 (1 sign, 2 exponent bits with bias 1, 1 mantissa bit):
  magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}, code = sign<<3 | index;
* ``E = floor(log2(max|x|)) - 2`` (2 = exponent of the largest E2M1 value);
  an all-zero block takes E = -127 (byte 0);
* ``v = x / 2^E`` (exact), rounded to the nearest E2M1 magnitude with ties to the
  even code (mantissa bit 0), magnitudes above 6 saturating to 6; the sign bit
  of x is kept, also when the magnitude rounds to 0.

GEMM: ``Y = sum_b 2^(Ea_b + Ew_b) * sum_{k in b} va*vw``. With ``I_b =
sum_{k in b} (2va)(2vw)`` (an exact integer), ``Y = sum_b I_b 2^(Ea+Ew-2)``.
"""
from __future__ import annotations

import numpy as np

from . import _native as nat

MX_BLOCK = 32
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """4-bit E2M1 codes (0..15) -> float64 values (the oracle's decoder)."""
    c = np.asarray(codes).astype(np.int64)
    table = np.array([nat.lib().orc_e2m1_value(i) for i in range(16)], dtype=np.float64)
    return table[c & 15]


def _f16_bits(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype != np.float16 or x.ndim != 2:
        raise TypeError("x must be a 2-D float16 array")
    return np.ascontiguousarray(x).view(np.uint16)


def mxfp4_quantize(x: np.ndarray):
    """MXFP4-quantize each row in blocks of 32 along K.

    Returns ``(codes, e8m0)``: codes uint8 [R, K] holding 0..15, scale bytes
    uint8 [R, K/32].
    """
    xb = _f16_bits(x)
    R, K = xb.shape
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    codes = np.empty((R, K), dtype=np.uint8)
    e8m0 = np.empty((R, K // MX_BLOCK), dtype=np.uint8)
    nat.check(nat.lib().orc_mxfp4_quantize(nat.ptr(xb), R, K, nat.ptr(codes), nat.ptr(e8m0), nat.threads))
    return codes, e8m0


def mxfp4_quantize_residual(x: np.ndarray):
    """Two-pass MXFP4 with the residual pass appended along K.

    Multi-Scale Dequant abstract (APEX4 page): the high-precision activation is
    decomposed into several low-precision components, each multiplied with the
    quantized weights by the native GEMM; for MXFP4 two passes. ARCQuant
    abstract (same page): the quantized residual is appended to the activation
    as extra channels of the reduction dimension, so one standard GEMM computes
    both terms. Reading taken (the plainest): the second pass is the same MX
    rule applied to the exact residual ``R = x - deq(Q(x))``, with its own
    per-block scale.

    Returns ``(codes, e8m0)`` of the augmented activation: codes uint8
    [R, 2K] = [Q(x) | Q(R)], scale bytes uint8 [R, 2K/32].
    """
    xb = _f16_bits(x)
    R, K = xb.shape
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    codes = np.empty((R, 2 * K), dtype=np.uint8)
    e8m0 = np.empty((R, 2 * K // MX_BLOCK), dtype=np.uint8)
    nat.check(nat.lib().orc_mxfp4_quantize_residual(nat.ptr(xb), R, K, nat.ptr(codes), nat.ptr(e8m0),
                                                    nat.threads))
    return codes, e8m0


def mxfp4_quantize_residual_tied(x: np.ndarray):
    """Two-pass MXFP4 with the second scale tied to the first: the reading under
    which the Multi-Scale Dequant abstract's "error bound 1/64 per block"
    holds. First pass: the smallest block exponent E1 with max|x| <= 6 2^E1
    (no element clips, so the residual r = x - deq(Q1(x)) satisfies
    |r| <= 2^E1); second pass: r at the fixed exponent E2 = E1 - 2 (no element
    clips either). Then |x - deq(Q1) - deq(Q2)| <= 2^(E1 - 3) = 2^(E1 + 3) / 64
    per element. An all-zero block takes E1 = -125. Returns ``(codes, e8m0)``
    as :func:`mxfp4_quantize_residual` ([Q1 | Q2] along K)."""
    xb = _f16_bits(x)
    R, K = xb.shape
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of 32")
    codes = np.empty((R, 2 * K), dtype=np.uint8)
    e8m0 = np.empty((R, 2 * K // MX_BLOCK), dtype=np.uint8)
    nat.check(nat.lib().orc_mxfp4_quantize_residual_tied(nat.ptr(xb), R, K, nat.ptr(codes), nat.ptr(e8m0),
                                                         nat.threads))
    return codes, e8m0


def mxfp4_append_copy(codes: np.ndarray, e8m0: np.ndarray):
    """The weight side of the appended-residual GEMM: each row's codes and
    scales twice along K, so that [Q(x) | Q(R)] @ [Q(w) | Q(w)]^T =
    Q(x) Q(w)^T + Q(R) Q(w)^T."""
    return np.concatenate([codes, codes], axis=1), np.concatenate([e8m0, e8m0], axis=1)


def mxfp4_dequantize(codes: np.ndarray, e8m0: np.ndarray) -> np.ndarray:
    """x_hat = v * 2^E in float64 (exact)."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    e = np.ascontiguousarray(e8m0, dtype=np.uint8)
    R, K = c.shape
    if K % MX_BLOCK or e.shape != (R, K // MX_BLOCK):
        raise ValueError("scale shape does not match the codes")
    out = np.empty((R, K), dtype=np.float64)
    nat.lib().orc_mxfp4_dequantize(nat.ptr(c), nat.ptr(e), R, K, nat.ptr(out))
    return out


def fp4_block_partials(ca: np.ndarray, cw: np.ndarray, block: int) -> np.ndarray:
    """``I[b] = (2 va_b) @ (2 vw_b)^T`` over blocks of ``block`` along K, int32 [K/block, M, N]."""
    a = np.ascontiguousarray(ca, dtype=np.uint8)
    w = np.ascontiguousarray(cw, dtype=np.uint8)
    M, K = a.shape
    N = w.shape[0]
    if w.shape[1] != K or K % block:
        raise ValueError(f"K mismatch or not a multiple of {block}")
    P = np.empty((K // block, M, N), dtype=np.int32)
    nat.check(nat.lib().orc_fp4_block_partials(nat.ptr(a), nat.ptr(w), M, N, K, block, nat.ptr(P),
                                               nat.threads))
    return P


def mxfp4_block_partials(ca: np.ndarray, cw: np.ndarray):
    """Yield ``(b, I_b)`` with ``I_b = (2 va_b) @ (2 vw_b)^T`` as int64 (exact)."""
    P = fp4_block_partials(ca, cw, MX_BLOCK)
    for b in range(P.shape[0]):
        yield b, P[b].astype(np.int64)


def mxfp4_gemm(ca: np.ndarray, ea: np.ndarray, cw: np.ndarray, ew: np.ndarray):
    """Block-scaled FP4 GEMM; returns ``(Y, T)`` in float64.

    ``Y[m,n] = sum_b I_b[m,n] * 2^(Ea[m,b] + Ew[n,b] - 2)`` in block order; each
    term is exact, ``T`` is the sum of their absolute values.
    """
    a = np.ascontiguousarray(ca, dtype=np.uint8)
    w = np.ascontiguousarray(cw, dtype=np.uint8)
    M, K = a.shape
    N = w.shape[0]
    e_a = np.ascontiguousarray(ea, dtype=np.uint8)
    e_w = np.ascontiguousarray(ew, dtype=np.uint8)
    if w.shape[1] != K or K % MX_BLOCK or e_a.shape != (M, K // MX_BLOCK) or e_w.shape != (N, K // MX_BLOCK):
        raise ValueError("scale shapes do not match")
    Y = np.empty((M, N), dtype=np.float64)
    T = np.empty((M, N), dtype=np.float64)
    nat.check(nat.lib().orc_mxfp4_gemm(nat.ptr(a), nat.ptr(e_a), nat.ptr(w), nat.ptr(e_w), M, N, K,
                                       nat.ptr(Y), nat.ptr(T), nat.threads))
    return Y, T
