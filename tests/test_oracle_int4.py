"""Pins for the INT4 oracle: quantizer and group-dequantized GEMM (CPU only).

Each check ties the oracle to something other than itself: exact rational
arithmetic, closed forms, invariants of the quantizer, library integer matmul,
or brute-force loops on tiny inputs.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from w4a4_quantized_gemm_quantize_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- exact helpers
def round_f32(r: Fraction) -> Fraction:
    """Nearest IEEE binary32 to the rational r, ties to even (no overflow)."""
    if r == 0:
        return Fraction(0)
    sign = -1 if r < 0 else 1
    r = abs(r)
    e = r.numerator.bit_length() - r.denominator.bit_length()
    if Fraction(2) ** e > r:
        e -= 1
    while Fraction(2) ** (e + 1) <= r:
        e += 1
    e = max(e, -126)                           # subnormal quantum below 2^-126
    quantum = Fraction(2) ** (e - 23)
    n = round(r / quantum)                      # Python rounds Fraction half-to-even
    return sign * n * quantum


def brute_quantize_group(xs):
    """Pure-Python exact-rational INT4 quantization of one group."""
    a = max(abs(Fraction(float(v))) for v in xs)
    if a == 0:
        return [0] * len(xs), Fraction(0)
    s = round_f32(a / 7)
    codes = []
    for v in xs:
        t = round_f32(Fraction(float(v)) / s)
        q = round(t)                            # half to even
        codes.append(max(-8, min(7, q)))
    return codes, s


# ---------------------------------------------------------------- quantizer
def test_binary32_division_matches_exact_rational():
    """The oracle's fl32 divisions equal exact-rational rounding (pins IEEE RNE)."""
    rng = np.random.default_rng(11)
    x = (rng.standard_t(3, size=(24, 64)) * rng.choice([1e-3, 1, 50], size=(24, 1))).astype(np.float16)
    codes, scales = oracle.int4_quantize(x, 32)
    for r in range(x.shape[0]):
        for j in range(2):
            grp = x[r, j * 32:(j + 1) * 32]
            bc, bs = brute_quantize_group(grp)
            assert Fraction(float(scales[r, j])) == bs
            assert list(codes[r, j * 32:(j + 1) * 32]) == bc


def test_exhaustive_fp16_against_exact_rational():
    """Every finite fp16 value |x| <= a quantized against a few anchors a."""
    allf = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16)   # +0 .. 65504
    allv = np.concatenate([allf, -allf[1:]])
    rng = np.random.default_rng(5)
    anchors = [np.float16(65504), np.float16(1.0), np.float16(2.0 ** -24),
               np.float16(3.14), rng.choice(allf[1:])]
    for a in anchors:
        vals = allv[np.abs(allv.astype(np.float32)) <= np.float32(a)]
        if vals.size > 3000:
            vals = rng.choice(vals, 3000, replace=False)
        n = (vals.size + 126) // 127
        grid = np.zeros(n * 127, dtype=np.float16)
        grid[:vals.size] = vals
        x = np.concatenate([np.full((n, 1), a, dtype=np.float16), grid.reshape(n, 127)], axis=1)
        codes, scales = oracle.int4_quantize(x, 128)
        s_exact = round_f32(Fraction(float(a)) / 7)
        assert np.all(scales[:, 0].astype(np.float64) == float(s_exact))
        for r in range(n):
            for c in range(128):
                t = round_f32(Fraction(float(x[r, c])) / s_exact)
                assert codes[r, c] == max(-8, min(7, round(t)))


def test_rne_tie_table():
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "int4_rne_ties.txt")) if ln.strip() and not ln.startswith("#")]
    xs = np.array([float(r[0]) for r in rows], dtype=np.float16)
    want = np.array([int(r[1]) for r in rows], dtype=np.int8)
    g = np.zeros(32, dtype=np.float16)
    g[0] = 7.0                                   # absmax 7 -> scale exactly 1
    x = np.tile(g, (len(xs), 1))
    x[:, 1] = xs
    codes, scales = oracle.int4_quantize(x, 32)
    assert np.all(scales == 1.0)
    assert np.array_equal(codes[:, 1], want)


def test_dequant_error_bound_and_code_range():
    """|q s - x| <= s/2 (1 + 2^-20) and codes in [-7, 7] (absmax/7 never reaches -8)."""
    x = synth.activations(64, 1024, dist="t3", seed=3)
    for g in (32, 64, 128, 256, 1024):
        codes, scales = oracle.int4_quantize(x, g)
        xh = oracle.int4_dequantize(codes, scales, g)
        s = np.repeat(scales.astype(np.float64), g, axis=1)
        err = np.abs(xh - x.astype(np.float64))
        assert np.all(err <= s / 2 * (1 + 2.0 ** -20))
        assert codes.min() >= -7 and codes.max() <= 7
        # the absmax element of each nonzero group maps to +-7
        absmax_codes = np.abs(codes.reshape(64, -1, g)).max(axis=2)
        assert np.all(absmax_codes[scales > 0] == 7)


def test_grid_aligned_round_trip():
    rng = np.random.default_rng(2)
    for e in (-20, -8, -1, 0, 3, 9):
        q = rng.integers(-7, 8, size=(8, 128))
        q[:, 0] = 7 * rng.choice([-1, 1], size=8)   # absmax exactly 7 * 2^e
        x = np.ldexp(q.astype(np.float64), e).astype(np.float16)
        assert np.array_equal(x.astype(np.float64), np.ldexp(q.astype(np.float64), e))
        codes, scales = oracle.int4_quantize(x, 128)
        assert np.all(scales == np.float32(2.0 ** e))
        assert np.array_equal(codes, q.astype(np.int8))


def test_zero_and_constant_groups():
    x = np.zeros((3, 256), dtype=np.float16)
    x[1, 128:] = 0.3
    x[2, :128] = -1e-7                             # fp16 subnormal
    codes, scales = oracle.int4_quantize(x, 128)
    assert scales[0, 0] == 0 and scales[0, 1] == 0 and scales[1, 0] == 0
    assert np.all(codes[0] == 0) and np.all(codes[1, :128] == 0)
    assert np.all(codes[1, 128:] == 7)
    assert np.all(codes[2, :128] == -7) and np.all(codes[2, 128:] == 0)
    assert scales[2, 0] == np.float32(np.float32(np.float16(-1e-7)) * -1) / np.float32(7)


def test_groups_are_independent_and_per_row():
    x = synth.activations(4, 512, dist="t3", seed=9)
    codes, scales = oracle.int4_quantize(x, 128)
    for r in range(4):
        for j in range(4):
            c1, s1 = oracle.int4_quantize(x[r:r + 1, j * 128:(j + 1) * 128].copy(), 128)
            assert s1[0, 0] == scales[r, j]
            assert np.array_equal(c1[0], codes[r, j * 128:(j + 1) * 128])


def test_rejects_bad_input():
    with pytest.raises(ValueError):
        oracle.int4_quantize(np.zeros((2, 100), np.float16), 128)
    with pytest.raises(ValueError):
        oracle.int4_quantize(np.array([[np.inf] * 128], np.float16), 128)
    with pytest.raises(TypeError):
        oracle.int4_quantize(np.zeros((2, 128), np.float32), 128)


# ---------------------------------------------------------------- packing
def test_pack_nibbles_generic_layout():
    u = np.array([[0, 15, 8, 9]], dtype=np.uint8)
    assert oracle.pack_nibbles(u).tolist() == [[0xF0, 0x98]]
    assert np.array_equal(oracle.unpack_nibbles_unsigned(oracle.pack_nibbles(u)), u)


def table_pack16(c, neg):
    """The INT4 word of 16 codes from an explicit bit-position table (a second,
    independent statement of the layout): returns (X, Y) as Python ints.
    X: c0..c4 magnitude at 6k..6k+2, sign at 6k+5; c5 magnitude bits 0, 1 at 30,
       31, sign at 3; c6..c9 magnitude bit 0 at 6(k-6)+4, sign at 6(k-6)+9;
       c10 magnitude bit 0 at 28.
    Y: c5 magnitude bit 2 at 0; c10 sign at 1; c6..c10 magnitude bits 1, 2 at
       6(k-6)+5, 6(k-6)+6; c11..c15 magnitude at 6(k-11)+2..+4, sign at 6(k-11)+7."""
    m = [abs(int(v)) for v in c]
    sg = [int(bool(v)) for v in neg]
    bit = lambda v, i: (v >> i) & 1
    x = y = 0
    for k in range(5):
        x |= m[k] << (6 * k) | sg[k] << (6 * k + 5)
    x |= bit(m[5], 0) << 30 | bit(m[5], 1) << 31 | sg[5] << 3
    y |= bit(m[5], 2) << 0
    for k in range(6, 10):
        x |= bit(m[k], 0) << (6 * (k - 6) + 4) | sg[k] << (6 * (k - 6) + 9)
    x |= bit(m[10], 0) << 28
    y |= sg[10] << 1
    for k in range(6, 11):
        y |= bit(m[k], 1) << (6 * (k - 6) + 5) | bit(m[k], 2) << (6 * (k - 6) + 6)
    for k in range(11, 16):
        y |= m[k] << (6 * (k - 11) + 2) | sg[k] << (6 * (k - 11) + 7)
    return x, y


def words(p):
    w = np.ascontiguousarray(p).view("<u4").reshape(-1)
    return [int(v) for v in w]


def test_pack_int4_bit_table_covers_each_bit_once():
    """Every one of the 64 bits belongs to exactly one (code, bit) pair."""
    seen = {}
    for k in range(16):
        for b in range(4):          # magnitude bits 0..2, sign as bit 3
            c = [0] * 16
            neg = [False] * 16
            if b < 3:
                c[k] = 1 << b
            else:
                neg[k] = True
            x, y = table_pack16(c, neg)
            v = x | y << 32
            assert v and v & (v - 1) == 0
            assert v not in seen
            seen[v] = (k, b)
    assert len(seen) == 64


def test_pack_int4_hand_computed_word():
    """c = [1, -2, 3, -4, 5, -6, 7, -7, 0, 1, 2, 3, -5, 6, -1, 4], summed by hand
    from the bit table:
    X = c0 0x1 + c1 0x80|0x800 + c2 0x3000 + c3 0x100000|0x800000 + c4 0x5000000
        + c5 (m1) 0x80000000 (sign) 0x8 + c6 (m0) 0x10 + c7 (m0) 0x400 (sign) 0x8000
        + c9 (m0) 0x400000 = 0x85D0BC99;
    Y = c5 (m2) 0x1 + c6 0x20|0x40 + c7 0x800|0x1000 + c10 (m1) 0x20000000
        + c11 0xC + c12 0x500|0x2000 + c13 0x18000 + c14 0x100000|0x2000000
        + c15 0x10000000 = 0x3211BD6D."""
    c = np.array([[1, -2, 3, -4, 5, -6, 7, -7, 0, 1, 2, 3, -5, 6, -1, 4]], dtype=np.int8)
    x, y = table_pack16(c[0], c[0] < 0)
    assert (x, y) == (0x85D0BC99, 0x3211BD6D)
    p = oracle.pack_int4(c, c < 0)
    assert words(p) == [x, y]
    codes, neg = oracle.unpack_int4(p)
    assert np.array_equal(codes, c) and np.array_equal(neg, c < 0)


def test_pack_int4_every_code_at_every_position():
    for k in range(16):
        for v in range(-7, 8):
            for negzero in ([False, True] if v == 0 else [v < 0]):
                c = np.zeros((1, 16), np.int8)
                neg = np.zeros((1, 16), bool)
                c[0, k] = v
                neg[0, k] = negzero
                assert words(oracle.pack_int4(c, neg)) == list(table_pack16(c[0], neg[0])), (k, v, negzero)


def test_pack_int4_random_words_match_bit_table():
    rng = np.random.default_rng(3)
    c = rng.integers(-7, 8, size=(4, 64)).astype(np.int8)
    neg = (c < 0) | ((c == 0) & (rng.random(c.shape) < 0.5))
    w = words(oracle.pack_int4(c, neg))
    for r in range(4):
        for j in range(4):
            assert w[8 * r + 2 * j: 8 * r + 2 * j + 2] == list(table_pack16(c[r, 16 * j:16 * j + 16],
                                                                            neg[r, 16 * j:16 * j + 16]))


def test_pack_int4_words_widen_to_fp6_e2m3():
    """Design property of the layout: S0 = X & ~FOLD_X, S1 = (X & FOLD_X) |
    (Y & FOLD_Y), S2 = Y & ~FOLD_Y is the 96-bit stream of OCP FP6 E2M3 fields
    (sign, 2 exponent bits, 3 mantissa bits, bias 1) of c0..c15, field k at bits
    6k..6k+5, whose values are exactly c_k / 8 (subnormals m/8); with E8M0
    scales 2^3 on both operands the matrix cores then multiply exact integers."""
    rng = np.random.default_rng(0)
    c = rng.integers(-7, 8, size=(5, 64)).astype(np.int8)
    neg = (c < 0) | ((c == 0) & (rng.random(c.shape) < 0.5))
    w = words(oracle.pack_int4(c, neg))
    fx, fy = 0x18618618, 0x61861861

    def e2m3(f):
        s, e, m = f >> 5, (f >> 3) & 3, f & 7
        v = (m / 8) if e == 0 else (1 + m / 8) * 2.0 ** (e - 1)
        return -v if s else v

    for u in range(len(w) // 2):
        x, y = w[2 * u], w[2 * u + 1]
        s0 = x & (0xFFFFFFFF ^ fx)
        s1 = (x & fx) | (y & fy)
        s2 = y & (0xFFFFFFFF ^ fy)
        stream = s0 | s1 << 32 | s2 << 64
        fields = [(stream >> (6 * k)) & 63 for k in range(16)]
        r, j = divmod(u, 4)
        assert [e2m3(f) for f in fields] == [float(v) / 8 for v in c[r, 16 * j:16 * j + 16]]
        assert all((f >> 3) & 3 == 0 for f in fields)          # subnormal encodings
        assert [f >> 5 for f in fields] == [int(b) for b in neg[r, 16 * j:16 * j + 16]]


def test_pack_int4_negative_zero_placement():
    """-0 keeps its sign bit: c5 (sign at X bit 3), c10 (Y bit 1), c13 (Y bit 19)."""
    for k, (xw, yw) in {5: (1 << 3, 0), 10: (0, 1 << 1), 13: (0, 1 << 19)}.items():
        z = np.zeros((1, 16), np.int8)
        negz = np.zeros((1, 16), bool)
        negz[0, k] = True
        assert words(oracle.pack_int4(z, negz)) == [xw, yw]


def test_pack_int4_round_trip_and_rejects():
    rng = np.random.default_rng(1)
    c = rng.integers(-7, 8, size=(7, 128)).astype(np.int8)
    neg = (c < 0) | ((c == 0) & (rng.random(c.shape) < 0.3))
    codes, n2 = oracle.unpack_int4(oracle.pack_int4(c, neg))
    assert np.array_equal(codes, c) and np.array_equal(n2, neg)
    with pytest.raises(ValueError):
        oracle.pack_int4(np.full((1, 16), -8, np.int8), np.ones((1, 16), bool))
    with pytest.raises(ValueError):
        oracle.pack_int4(np.ones((1, 16), np.int8), np.ones((1, 16), bool))
    with pytest.raises(ValueError):
        oracle.pack_int4(np.ones((1, 8), np.int8), np.zeros((1, 8), bool))


def test_sign_bits_follow_input():
    x = np.array([[0.0, -0.0, 1.0, -1.0, -1e-8, 1e-8, 3.0, -3.0]], np.float16)
    assert oracle.int4_sign_bits(x).tolist() == [[False, True, False, True, True, False, False, True]]


# ---------------------------------------------------------------- GEMM
def brute_gemm(qa, sa, ga, qw, sw, gw):
    """Per-element dequantize-multiply-sum with exact rationals."""
    M, K = qa.shape
    N = qw.shape[0]
    Y = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += (int(qa[m, k]) * Fraction(float(sa[m, k // ga]))
                        * int(qw[n, k]) * Fraction(float(sw[n, k // gw])))
            Y[m][n] = acc
    return Y


@pytest.mark.parametrize("ga,gw", [(16, 16), (32, 16), (16, 64), (64, 64)])
def test_gemm_brute_force_tiny(ga, gw):
    rng = np.random.default_rng(ga * 7 + gw)
    M, N, K = 3, 5, 64
    xa = (rng.standard_normal((M, K)) * 2).astype(np.float16)
    xw = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    qa, sa = oracle.int4_quantize(xa, ga)
    qw, sw = oracle.int4_quantize(xw, gw)
    Y, T = oracle.w4a4_gemm(qa, sa, ga, qw, sw, gw)
    B = brute_gemm(qa, sa, ga, qw, sw, gw)
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(Y[m, n]) - B[m][n]) <= Fraction(T[m, n]) * Fraction(1, 2 ** 48)
    # partials against a plain int loop
    g = min(ga, gw)
    for b, P in oracle.w4a4_block_partials(qa, qw, g):
        for m in range(M):
            for n in range(N):
                ref = sum(int(qa[m, k]) * int(qw[n, k]) for k in range(b * g, (b + 1) * g))
                assert P[m, n] == ref


def test_gemm_all_scales_one_is_integer_matmul():
    rng = np.random.default_rng(4)
    M, N, K, g = 9, 13, 256, 128
    qa = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    qw = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    qa[:, ::g] = 7
    qw[:, ::g] = -7
    xa = qa.astype(np.float16)
    xw = qw.astype(np.float16)
    qa2, sa = oracle.int4_quantize(xa, g)
    qw2, sw = oracle.int4_quantize(xw, g)
    assert np.all(sa == 1) and np.all(sw == 1)
    assert np.array_equal(qa2, qa) and np.array_equal(qw2, qw)
    Y, T = oracle.w4a4_gemm(qa2, sa, g, qw2, sw, g)
    ref = qa.astype(np.int64) @ qw.astype(np.int64).T            # integer routine
    assert np.array_equal(Y, ref.astype(np.float64))


def test_gemm_constant_closed_form():
    M, N, K, g = 4, 6, 512, 128
    c, d = np.float16(0.75), np.float16(-0.0123)
    qa, sa = oracle.int4_quantize(np.full((M, K), c), g)
    qw, sw = oracle.int4_quantize(np.full((N, K), d), g)
    Y, T = oracle.w4a4_gemm(qa, sa, g, qw, sw, g)
    s_a = np.float32(np.float32(c) / np.float32(7))
    s_w = np.float32(np.float32(abs(d)) / np.float32(7))
    want = -(K // g) * 49 * g * float(s_a) * float(s_w)
    assert np.all(Y == want) and np.all(T == -want)


def test_gemm_per_token_reduces_to_scaled_integer_matmul():
    rng = np.random.default_rng(8)
    M, N, K = 7, 11, 384
    xa = rng.standard_normal((M, K)).astype(np.float16)
    xw = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    qa, sa = oracle.int4_quantize(xa, K)
    qw, sw = oracle.int4_quantize(xw, K)
    Y, _ = oracle.w4a4_gemm(qa, sa, K, qw, sw, K)
    I = qa.astype(np.int64) @ qw.astype(np.int64).T
    ref = sa[:, 0:1].astype(np.float64) * sw[:, 0].astype(np.float64)[None, :] * I
    assert np.array_equal(Y, ref)


@pytest.mark.parametrize("ga,gw", [(128, 128), (64, 128), (512, 128), (1024, 128)])
def test_gemm_matches_dequantize_then_matmul(ga, gw):
    M, N, K = 32, 48, 1024
    xa = synth.activations(M, K, dist="t3", seed=1)
    xw = synth.weights(N, K, seed=1)
    qa, sa = oracle.int4_quantize(xa, ga)
    qw, sw = oracle.int4_quantize(xw, gw)
    Y, T = oracle.w4a4_gemm(qa, sa, ga, qw, sw, gw)
    ref = oracle.int4_dequantize(qa, sa, ga) @ oracle.int4_dequantize(qw, sw, gw).T
    assert np.all(np.abs(Y - ref) <= 1e-12 * T + 1e-300)
    assert np.all(T >= np.abs(Y))
    # non-square shapes would expose a transposed operand
    assert Y.shape == (M, N)


def test_gemm_rows_is_a_row_slice():
    M, N, K = 20, 24, 256
    xa = synth.activations(M, K, dist="t3", seed=2)
    xw = synth.weights(N, K, seed=2)
    qa, sa = oracle.int4_quantize(xa, 128)
    qw, sw = oracle.int4_quantize(xw, 128)
    Y, T = oracle.w4a4_gemm(qa, sa, 128, qw, sw, 128)
    rows = [0, 5, 19]
    Yr, Tr = oracle.w4a4_gemm_rows(qa, sa, 128, qw, sw, 128, rows)
    assert np.array_equal(Yr, Y[rows]) and np.array_equal(Tr, T[rows])


def test_gemm_rejects_non_nested_groups():
    qa = np.zeros((2, 384), np.int8)
    with pytest.raises(ValueError):
        oracle.w4a4_gemm(qa, np.zeros((2, 3), np.float32), 128, qa, np.zeros((2, 2), np.float32), 192)
