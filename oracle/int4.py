"""INT4 symmetric group quantization and the W4A4 group-dequantized GEMM (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages fix ("APEX4: Efficient Pure W4A4 LLM Inference via Intra-SM
Compute Rebalancing", abstract, three copies on the pages): 4-bit weights AND
4-bit activations, groups of 128 along the reduction axis ("W4A4-g128"), a pure
INT4 matrix product whose per-group results are then dequantized by the vector
units ("group dequantization ... on CUDA Cores"), and a mixed-granularity mode in
which the activation group size differs from the weight one. They give no
quantization formula, rounding mode, scale type or memory layout. The readings
taken here:

* symmetric, no zero point; per row and per group of ``g`` consecutive K
  elements: ``a = max|x|``, ``s = fl32(a / 7)``, ``q = clamp(rne(fl32(x / s)),
  -8, 7)``; an all-zero group has ``s = 0`` and codes 0;
* scales are IEEE binary32; divisions are correctly rounded binary32 (the
  precision the kernel makes the integer decision in); ties round to even;
* packed layout (the pages give none): row-major, K contiguous, 4 bits per
  code, sign-magnitude. The symmetric rule only yields codes in [-7, 7] (the
  clamp at -8 never fires), so a sign bit and a 3-bit magnitude hold every code.
  A code's sign bit is the sign bit of its input value (so a negative input that
  rounds to 0 is stored as -0). Each 8-byte unit holds the 16 codes c0..c15 of
  k = 16j .. 16j+15 as two little-endian 32-bit words X, Y, defined through the
  96-bit stream S of 6-bit fields ``f_k = sign_k << 5 | |c_k|`` at bits 6k..6k+5
  (f_k is the OCP FP6 E2M3 encoding of the subnormal +-|c_k|/8, so its bits 3
  and 4 are zero). With S0, S1, S2 the 32-bit words of S,
  ``X = S0 | (S1 & FOLD_X)`` and ``Y = S2 | (S1 & FOLD_Y)``: FOLD_X marks the
  bits of a word at positions 3, 4 mod 6 (where S0 is zero), FOLD_Y those at
  0, 5 mod 6 (where S2 is zero), and together they cover every bit that S1
  can have set. The kernel rebuilds S with two ANDs and an AND-OR.;
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


def _check_group(K: int, group: int) -> None:
    if group <= 0 or K % group != 0:
        raise ValueError(f"group {group} must divide K={K}")


def int4_quantize(x: np.ndarray, group: int):
    """Symmetric INT4 quantization of each row in groups of ``group`` along K.

    Returns ``(codes, scales)``: codes int8 [R, K] in [-8, 7], scales float32
    [R, K/group]. Follows the steps listed in the module docstring, in order.
    """
    x = np.asarray(x)
    if x.dtype != np.float16 or x.ndim != 2:
        raise TypeError("x must be a 2-D float16 array")
    R, K = x.shape
    _check_group(K, group)
    xf = x.astype(np.float32)                      # fp16 -> fp32 is exact
    if not np.isfinite(xf).all():
        raise ValueError("NaN/Inf inputs are outside the quantizer's contract")
    xg = xf.reshape(R, K // group, group)
    a = np.abs(xg).max(axis=2)                     # exact
    s = (a / np.float32(7.0)).astype(np.float32)   # one binary32 division, RNE
    with np.errstate(divide="ignore", invalid="ignore"):
        t = xg / s[:, :, None]                     # binary32 division, RNE
    q = np.rint(t)                                 # round half to even
    q = np.where(s[:, :, None] == 0, np.float32(0), q)
    q = np.clip(q, -8, 7).astype(np.int8)
    return q.reshape(R, K), s


def int4_dequantize(codes: np.ndarray, scales: np.ndarray, group: int) -> np.ndarray:
    """x_hat = q * s in float64 (exact: 4-bit times 24-bit significands)."""
    R, K = codes.shape
    _check_group(K, group)
    s = np.repeat(scales.astype(np.float64), group, axis=1)
    return codes.astype(np.float64) * s


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Generic 4-bit field packing: two fields per byte, even k in the low nibble.

    Used for MXFP4 E2M1 codes (fields 0..15); INT4 codes use :func:`pack_int4`.
    """
    c = np.asarray(codes)
    if c.ndim != 2 or c.shape[1] % 2:
        raise ValueError("codes must be 2-D with an even number of columns")
    u = (c.astype(np.int16) & 0xF).astype(np.uint8)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def unpack_nibbles_unsigned(packed: np.ndarray) -> np.ndarray:
    """Inverse of :func:`pack_nibbles` giving the raw 4-bit fields 0..15."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty((p.shape[0], p.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


FOLD_X = sum(1 << q for q in range(32) if q % 6 in (3, 4))   # 0x18618618
FOLD_Y = sum(1 << q for q in range(32) if q % 6 in (0, 5))   # 0x61861861
_MASK32 = 0xFFFFFFFF


def _stream_words(fields: np.ndarray):
    """The 96-bit stream of 16 six-bit fields [..., 16] as three uint64 arrays
    holding its 32-bit words S0, S1, S2 (field k at stream bits 6k..6k+5)."""
    words = []
    for d in range(3):
        acc = np.zeros(fields.shape[:-1], dtype=np.uint64)
        for k in range(16):
            sh = 6 * k - 32 * d
            if -6 < sh < 32:
                f = fields[..., k].astype(np.uint64)
                acc |= (f << np.uint64(sh)) if sh >= 0 else (f >> np.uint64(-sh))
        words.append(acc & np.uint64(_MASK32))
    return words


def pack_int4(codes: np.ndarray, negative: np.ndarray) -> np.ndarray:
    """Sign-magnitude INT4 packing (layout in the module docstring).

    ``codes``: int [R, K] in [-7, 7], K a multiple of 16; ``negative``: bool
    [R, K], the sign bit of each code (must agree with the code where it is not
    zero). Returns uint8 [R, K/2].
    """
    c = np.asarray(codes).astype(np.int16)
    neg = np.asarray(negative, dtype=bool)
    if c.ndim != 2 or c.shape[1] % 16 or neg.shape != c.shape:
        raise ValueError("codes and signs must be 2-D, equal shapes, K a multiple of 16")
    if np.abs(c).max(initial=0) > 7:
        raise ValueError("sign-magnitude INT4 holds codes in [-7, 7]")
    if np.any((c != 0) & (neg != (c < 0))):
        raise ValueError("sign bits disagree with nonzero codes")
    R, K = c.shape
    fields = ((neg.astype(np.uint8) << 5) | np.abs(c).astype(np.uint8)).reshape(R, K // 16, 16)
    s0, s1, s2 = _stream_words(fields)
    x = s0 | (s1 & np.uint64(FOLD_X))
    y = s2 | (s1 & np.uint64(FOLD_Y))
    out = np.empty((R, K // 16, 2), dtype="<u4")
    out[..., 0] = x.astype(np.uint32)
    out[..., 1] = y.astype(np.uint32)
    return out.reshape(R, K // 8).view(np.uint8).reshape(R, K // 2)


def unpack_int4(packed: np.ndarray):
    """Inverse of :func:`pack_int4`: ``(codes int8 [R, K], negative bool [R, K])``."""
    p = np.asarray(packed, dtype=np.uint8)
    if p.ndim != 2 or p.shape[1] % 8:
        raise ValueError("packed rows must hold whole 8-byte units")
    R, H = p.shape
    w = np.ascontiguousarray(p).view("<u4").reshape(R, H // 8, 2).astype(np.uint64)
    x, y = w[..., 0], w[..., 1]
    s0 = x & np.uint64(_MASK32 ^ FOLD_X)
    s1 = (x & np.uint64(FOLD_X)) | (y & np.uint64(FOLD_Y))
    s2 = y & np.uint64(_MASK32 ^ FOLD_Y)
    stream = [s0, s1, s2]
    fields = np.empty((R, H // 8, 16), dtype=np.uint64)
    for k in range(16):
        d, o = divmod(6 * k, 32)
        f = stream[d] >> np.uint64(o)
        if o > 26:
            f |= stream[d + 1] << np.uint64(32 - o)
        fields[..., k] = f & np.uint64(63)
    mag = (fields & np.uint64(7)).astype(np.int16)
    sg = (fields >> np.uint64(5)).astype(bool)
    codes = np.where(sg, -mag, mag).astype(np.int8)
    return codes.reshape(R, 2 * H), sg.reshape(R, 2 * H)


def int4_sign_bits(x: np.ndarray) -> np.ndarray:
    """Sign bit stored with each INT4 code: the sign bit of the fp16 input."""
    return np.signbit(np.asarray(x))


def _nested_groups(K: int, g_a: int, g_w: int) -> int:
    _check_group(K, g_a)
    _check_group(K, g_w)
    g = min(g_a, g_w)
    if max(g_a, g_w) % g:
        raise ValueError("activation and weight groups must nest")
    return g


def w4a4_block_partials(qa: np.ndarray, qw: np.ndarray, g: int):
    """Yield ``(b, P_b)`` with ``P_b = qa[:, block b] @ qw[:, block b]^T`` (int64).

    The matrix product of the integer codes is taken in float64 with a library
    matmul: every product and partial sum is an integer below 2^53 in magnitude,
    so it is exact whatever order the library sums in.
    """
    R, K = qa.shape
    _check_group(K, g)
    if qw.shape[1] != K:
        raise ValueError("K mismatch")
    for b in range(K // g):
        A = qa[:, b * g:(b + 1) * g].astype(np.float64)
        W = qw[:, b * g:(b + 1) * g].astype(np.float64)
        P = A @ W.T
        yield b, P.astype(np.int64)


def w4a4_gemm(qa: np.ndarray, sa: np.ndarray, g_a: int,
              qw: np.ndarray, sw: np.ndarray, g_w: int):
    """Group-dequantized INT4 GEMM; returns ``(Y, T)`` in float64.

    ``Y[m,n] = sum_b s_a[m, b g/g_a] * s_w[n, b g/g_w] * P_b[m,n]`` summed in
    block order; ``T`` is the same sum of absolute values.
    """
    M, K = qa.shape
    N = qw.shape[0]
    g = _nested_groups(K, g_a, g_w)
    if sa.shape != (M, K // g_a) or sw.shape != (N, K // g_w):
        raise ValueError("scale shapes do not match the groups")
    sa64 = sa.astype(np.float64)
    sw64 = sw.astype(np.float64)
    Y = np.zeros((M, N), dtype=np.float64)
    T = np.zeros((M, N), dtype=np.float64)
    for b, P in w4a4_block_partials(qa, qw, g):
        scale = sa64[:, (b * g) // g_a][:, None] * sw64[:, (b * g) // g_w][None, :]
        term = scale * P
        Y += term
        T += np.abs(term)
    return Y, T


def w4a4_gemm_rows(qa: np.ndarray, sa: np.ndarray, g_a: int,
                   qw: np.ndarray, sw: np.ndarray, g_w: int, rows) -> tuple:
    """:func:`w4a4_gemm` restricted to the listed output rows (same arithmetic)."""
    rows = np.asarray(rows, dtype=np.int64)
    return w4a4_gemm(qa[rows], sa[rows], g_a, qw, sw, g_w)
