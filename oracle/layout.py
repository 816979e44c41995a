"""Storage layouts of codes and scales (oracle side): byte permutations only.

TEST INFRASTRUCTURE ONLY (see the package docstring). Nothing here decides a
code or a scale: the C++ oracle computes codes as plain integers and scales as
plain numbers, and these functions only place them in memory the way the C
ABI documents, so GPU bytes can be compared bit for bit. Each layout is pinned
by a table of bit positions in ``tests/test_oracle_int4.py`` /
``tests/test_layout.py``.

* Two's-complement nibbles (the canonical layout of INT4 codes and of 4-bit
  E2M1 fields): two codes per byte, the even k in the low nibble.
* The GEMM's INT4 operand layout: sign-magnitude codes in [-7, 7] (the sign
  bit is that of the input value, so a negative input that rounds to 0 is
  stored as -0), each 8-byte unit holding the codes c0..c15 of 16 consecutive
  k as two little-endian 32-bit words X, Y, defined through the 96-bit stream
  S of 6-bit fields ``f_k = sign_k << 5 | |c_k|`` at bits 6k..6k+5 (the OCP
  FP6 E2M3 encoding of the subnormal +-|c_k|/8, whose bits 3 and 4 are zero).
  With S0, S1, S2 the 32-bit words of S: ``X = S0 | (S1 & FOLD_X)``,
  ``Y = S2 | (S1 & FOLD_Y)``; FOLD_X marks positions 3, 4 mod 6 (where S0 is
  zero), FOLD_Y positions 0, 5 mod 6 (where S2 is zero).
* Group-major INT4 scales: ``[K/g][rows]``, the transpose of the oracle's
  row-major ``[rows][K/g]``.
* E8M0 (MXFP4) and E4M3 (NVFP4) scale panels of 256 k, as the C header
  states them (offset functions below).
"""
from __future__ import annotations

import numpy as np

FOLD_X = sum(1 << q for q in range(32) if q % 6 in (3, 4))   # 0x18618618
FOLD_Y = sum(1 << q for q in range(32) if q % 6 in (0, 5))   # 0x61861861
_MASK32 = 0xFFFFFFFF


# ------------------------------------------------------------ nibbles

def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Two 4-bit fields per byte, even k in the low nibble. Fields are the low
    4 bits of each code: two's complement for INT4 codes in [-8, 7], the raw
    field for E2M1 codes 0..15."""
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


def pack_int4_twos(codes: np.ndarray) -> np.ndarray:
    """Canonical INT4 storage: two's-complement nibbles, even k low."""
    c = np.asarray(codes)
    if c.size and (c.min() < -8 or c.max() > 7):
        raise ValueError("INT4 codes lie in [-8, 7]")
    return pack_nibbles(c)


def unpack_int4_twos(packed: np.ndarray) -> np.ndarray:
    """Inverse of :func:`pack_int4_twos`: int8 codes in [-8, 7]."""
    u = unpack_nibbles_unsigned(packed).astype(np.int16)
    return np.where(u >= 8, u - 16, u).astype(np.int8)


# --------------------------------------------- the GEMM's INT4 operand layout

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
    """The GEMM's sign-magnitude INT4 layout (module docstring).

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
    """Sign bit stored with each INT4 code in the GEMM layout: the sign bit of
    the fp16 input."""
    return np.signbit(np.asarray(x))


# --------------------------------------------------------------- scales

def group_major(scales_rows: np.ndarray) -> np.ndarray:
    """Row-major INT4 scales [rows][K/g] -> the GEMM's group-major [K/g][rows]."""
    return np.ascontiguousarray(np.asarray(scales_rows).T)


def e8m0_panel_offsets(rows: int, K: int) -> np.ndarray:
    """Byte offset of the E8M0 scale of (row r, block b) in the 256-k panel
    layout: panel p = b // 8 holds, row after row, ``w_p = min(8, K/32 - 8p)``
    bytes per row, the even blocks of the panel first; returns int64 [rows, K/32]."""
    nb = K // 32
    off = np.empty((rows, nb), dtype=np.int64)
    for b in range(nb):
        p, j = divmod(b, 8)
        w = min(8, nb - 8 * p)
        pos = j // 2 if j % 2 == 0 else (w + 1) // 2 + j // 2
        off[:, b] = 8 * rows * p + w * np.arange(rows) + pos
    return off


def e4m3_panel_offsets(rows: int, K: int) -> np.ndarray:
    """Byte offset of the E4M3 scale of (row r, block b) in the 256-k panel
    layout: panel p = b // 16 holds 16 bytes per row, row after row, blocks
    in the order 0,1,4,5,8,9,12,13,2,3,6,7,10,11,14,15; returns int64 [rows, K/16]."""
    order = [0, 1, 4, 5, 8, 9, 12, 13, 2, 3, 6, 7, 10, 11, 14, 15]
    pos_of = {blk: i for i, blk in enumerate(order)}
    nb = K // 16
    off = np.empty((rows, nb), dtype=np.int64)
    for b in range(nb):
        p, j = divmod(b, 16)
        off[:, b] = 16 * rows * p + 16 * np.arange(rows) + pos_of[j]
    return off


def to_panels(rows_bytes: np.ndarray, offsets: np.ndarray) -> np.ndarray:
    """Row-major scale bytes [rows, nb] -> the flat panel layout given by ``offsets``."""
    out = np.empty(rows_bytes.size, dtype=np.uint8)
    out[offsets.reshape(-1)] = np.asarray(rows_bytes, dtype=np.uint8).reshape(-1)
    return out


def from_panels(flat: np.ndarray, offsets: np.ndarray) -> np.ndarray:
    """The flat panel layout -> row-major [rows, nb] (inverse of :func:`to_panels`)."""
    return np.asarray(flat).reshape(-1)[offsets]
