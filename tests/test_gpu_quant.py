"""GPU parity of the quantization kernels against the oracle: codes and scales
must match bit for bit (INT4 and MXFP4), on the workload shapes, ragged and
strided inputs, every supported group size, and exhaustive fp16 sweeps."""
import numpy as np
import pytest

import oracle
from w4a4_quantized_gemm_quantize_amd import synth
from helpers import dev, host

pytestmark = pytest.mark.gpu


def ops():
    from w4a4_quantized_gemm_quantize_amd import ops as o
    return o


def int4_check(x16, group, ldx_pad=0):
    M, K = x16.shape
    if ldx_pad:
        buf = np.zeros((M, K + ldx_pad), np.float16)
        buf[:, :K] = x16
        xt = dev(buf)[:, :K]
    else:
        xt = dev(x16)
    q, s = ops().w4a4_quantize_act(xt, group)
    codes, scales = oracle.int4_quantize(x16, group)
    want = oracle.pack_int4(codes, oracle.int4_sign_bits(x16))
    bad = np.argwhere(host(q) != want)
    assert bad.size == 0, f"codes differ at {bad[:5].tolist()} (M={M} K={K} g={group})"
    gs = np.ascontiguousarray(host(s).T)   # group-major on the device
    assert np.array_equal(gs.view(np.uint32), scales.view(np.uint32)), f"scales differ (M={M} K={K} g={group})"


def test_int4_tiny_config():
    int4_check(synth.activations(16, 256, dist="normal", seed=0), 128)


@pytest.mark.parametrize("group", [64, 128, 256, 512, "K"])
def test_int4_groups_ragged_rows(group):
    M, K = 37, 2048
    g = K if group == "K" else group
    int4_check(synth.activations(M, K, dist="t3", seed=1), g)


def test_int4_strided_rows_and_per_token_long_rows():
    int4_check(synth.activations(9, 1024, dist="t3", seed=2), 128, ldx_pad=64)
    int4_check(synth.activations(5, 28672, dist="t3", seed=3), 28672)
    int4_check(synth.activations(3, 1008, dist="t3", seed=3), 1008)     # per token, K % 128 != 0


def test_int4_zero_rows_and_groups():
    x = synth.activations(8, 512, dist="t3", seed=4)
    x[2] = 0
    x[5, 128:256] = 0
    x[6, :] = np.float16(-0.0)
    x[7, 3] = np.float16(-0.0)                 # -0 inside groups whose absmax is not 0:
    x[7, 130:140] = np.float16(-0.0)           # the code keeps the input's sign bit
    x[1, 64:128] = np.float16(-0.0)            # a whole g = 64 group of -0 in a nonzero row
    x[0, 5] = np.float16(-2.0 ** -24)          # tiny negatives that round to code -0
    x[0, 6] = np.float16(2.0 ** -24)
    for g in (64, 128, 512):
        int4_check(x, g)
    int4_check(x[:, :496], 496)                # per token, K % 32 == 16 (16-element tail)


def test_int4_exhaustive_fp16():
    """Every finite fp16 value against 64 absmax anchors, groups of 128."""
    rng = np.random.default_rng(0)
    allf = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16)
    allv = np.concatenate([allf, -allf[1:]])
    anchors = np.concatenate([
        np.array([65504, 1, 2.0 ** -24, 2.0 ** -14, 7, 0.5, 3.140625, 1000], np.float16),
        rng.choice(allf[1:], 56)]).astype(np.float16)
    rows = []
    for a in anchors:
        vals = allv[np.abs(allv.astype(np.float32)) <= np.float32(a)]
        n = (vals.size + 126) // 127
        pad = np.zeros(n * 127, np.float16)
        pad[:vals.size] = vals
        rows.append(np.concatenate([np.full((n, 1), a, np.float16), pad.reshape(n, 127)], axis=1))
    x = np.concatenate(rows)                 # one group of 128 per row
    n8 = x.shape[0] - x.shape[0] % 8         # 8 groups per 1024-wide row
    int4_check(x[:n8].reshape(-1, 1024), 128)
    if x.shape[0] > n8:
        int4_check(x[n8:], 128)


@pytest.mark.parametrize("name", ["llama2_7b_w13", "llama2_7b_w2", "llama2_70b_w13", "llama2_70b_w2"])
def test_int4_workload_activations_sampled(name):
    """Full-size activation quantization; bit-exact on a seeded row sample."""
    wl = synth.WORKLOADS[name]
    M, K = wl["M"], wl["K"]
    x = synth.activations(M, K, dist=wl["dist"], seed=0)
    q, s = ops().w4a4_quantize_act(dev(x), 128)
    rows = synth.sample_rows(M, 64, seed=1)
    codes, scales = oracle.int4_quantize(x[rows], 128)
    assert np.array_equal(host(q)[rows], oracle.pack_int4(codes, oracle.int4_sign_bits(x[rows])))
    assert np.array_equal(np.ascontiguousarray(host(s)[:, rows].T).view(np.uint32), scales.view(np.uint32))


def test_int4_rows_beyond_one_grid_dimension():
    """More row blocks than one grid dimension holds (65535): the kernel loops
    over the rest. Bit-exact on sampled rows and the last rows."""
    for g, K, M in ((128, 128, 65535 * 16 + 40), (512, 512, 65535 * 4 + 12)):
        x = synth.bulk_normal(M, K, seed=8)
        q, s = ops().w4a4_quantize_act(dev(x), g)
        rows = np.concatenate([synth.sample_rows(M, 48, seed=2), np.arange(M - 80, M)])
        codes, scales = oracle.int4_quantize(x[rows], g)
        assert np.array_equal(host(q)[rows], oracle.pack_int4(codes, oracle.int4_sign_bits(x[rows]))), (g, M)
        assert np.array_equal(np.ascontiguousarray(host(s)[:, rows].T).view(np.uint32), scales.view(np.uint32)), (g, M)
        del x, q, s


# ------------------------------------------------------------------ MXFP4
def mx_check(x16, ldx_pad=0):
    R, K = x16.shape
    if ldx_pad:
        buf = np.zeros((R, K + ldx_pad), np.float16)
        buf[:, :K] = x16
        xt = dev(buf)[:, :K]
    else:
        xt = dev(x16)
    q, e = ops().mxfp4_quantize(xt)
    codes, e8 = oracle.mxfp4_quantize(x16)
    assert np.array_equal(oracle.from_panels(host(e), oracle.e8m0_panel_offsets(R, K)), e8), f"E8M0 differ (R={R} K={K})"
    gq = host(q)
    want = oracle.pack_nibbles(codes)   # E2M1 fields, even k low
    bad = np.argwhere(gq != want)
    assert bad.size == 0, f"codes differ at {bad[:5].tolist()} (R={R} K={K})"


def test_mxfp4_exhaustive_fp16():
    rng = np.random.default_rng(1)
    allf = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16)
    allv = np.concatenate([allf, -allf])
    perm = rng.permutation(allv)
    perm = np.concatenate([perm, np.zeros((-perm.size) % 31, np.float16)])
    blocks = perm.reshape(-1, 31)
    anchors = np.abs(blocks.astype(np.float32)).max(axis=1) * rng.choice([1, 1.5, 3, 1000], size=blocks.shape[0])
    anchors = np.clip(anchors, 0, 65504).astype(np.float16)
    x = np.concatenate([anchors[:, None], blocks], axis=1).reshape(-1)
    x = np.concatenate([x, np.zeros((-x.size) % 1024, np.float16)]).reshape(-1, 1024)
    mx_check(x)


def test_mxfp4_every_value_under_every_block_exponent():
    """Every pair (x, E) of a finite fp16 value and a block exponent it can be
    quantized under. A block's exponent depends only on the binade of its
    absmax a (E = floor(log2 a) - 2, E in [-26, 13] for fp16), and x can share
    a block with exponent E exactly when |x| <= a; so for each E the block
    absmax is the largest fp16 of binade E + 2 and the other 31 elements sweep
    every fp16 of magnitude up to it, both signs."""
    f16 = np.arange(1, 0x7C00, dtype=np.uint16)                # positive finite fp16, increasing
    v = f16.view(np.float16).astype(np.float64)
    blocks = []
    for E in range(-26, 14):
        in_binade = (v >= 2.0 ** (E + 2)) & (v < 2.0 ** (E + 3))
        a_bits = int(f16[in_binade].max())
        xs = np.concatenate([np.arange(0, a_bits + 1, dtype=np.uint16),
                             np.arange(0, a_bits + 1, dtype=np.uint16) | np.uint16(0x8000)])
        n = -(-xs.size // 31)
        pad = np.full(n * 31, 0, np.uint16)
        pad[:xs.size] = xs
        b = np.empty((n, 32), np.uint16)
        b[:, 0] = a_bits
        b[:, 1:] = pad.reshape(n, 31)
        blocks.append(b)
    x = np.concatenate(blocks)
    x = np.concatenate([x, np.zeros(((-x.shape[0]) % 32, 32), np.uint16)]).reshape(-1, 1024).view(np.float16)
    e8 = oracle.mxfp4_quantize(x)[1].reshape(-1)
    assert set(np.unique(e8[e8 > 0]).tolist()) == set(range(127 - 26, 127 + 14))   # all 40 exponents occur
    mx_check(x)


def test_mxfp4_shapes():
    mx_check(synth.activations(16, 256, dist="normal", seed=0))
    mx_check(synth.activations(33, 3584, dist="t3", seed=5), ldx_pad=32)
    x = synth.activations(7, 18944, dist="t3", seed=6)
    x[3, :64] = 0
    mx_check(x)
    mx_check(synth.weights(40, 3584, seed=7))
    mx_check(synth.activations(19, 1120, dist="t3", seed=9))    # last panel 3 blocks wide
    mx_check(synth.activations(5, 96, dist="t3", seed=10))      # one panel, 3 blocks


def test_mxfp4_rows_beyond_one_grid_dimension():
    R, K = 65535 * 8 + 24, 64
    x = synth.bulk_normal(R, K, seed=11)
    q, e = ops().mxfp4_quantize(dev(x))
    rows = np.concatenate([synth.sample_rows(R, 48, seed=3), np.arange(R - 40, R)])
    codes, e8 = oracle.mxfp4_quantize(x[rows])
    assert np.array_equal(oracle.from_panels(host(e), oracle.e8m0_panel_offsets(R, K))[rows], e8)
    assert np.array_equal(host(q)[rows], oracle.pack_nibbles(codes))


def _anchor_groups(lo, hi):
    """Groups [a, x_1..x_127] covering, for each anchor bit pattern i in [lo, hi),
    every fp16 x with |x| <= a (a = the fp16 with bits i), zero-padded."""
    parts = []
    for i in range(lo, hi):
        xs = np.concatenate([np.arange(0, i + 1, dtype=np.uint16),
                             np.arange(1, i + 1, dtype=np.uint16) | np.uint16(0x8000)])
        n = -(-xs.size // 127)
        pad = np.zeros(n * 127, np.uint16)
        pad[:xs.size] = xs
        g = np.empty((n, 128), np.uint16)
        g[:, 0] = i
        g[:, 1:] = pad.reshape(n, 127)
        parts.append(g)
    g = np.concatenate(parts)
    g = np.concatenate([g, np.zeros(((-g.shape[0]) % 8, 128), np.uint16)])
    return g.reshape(-1, 1024).view(np.float16)


def test_int4_exhaustive_every_absmax_x_pair():
    """Every pair (a, x) of finite fp16 values with |x| <= a, a > 0: the scale
    depends only on a and the code only on (x, scale), so this covers every
    scale the quantizer can produce against every input it can see."""
    top = 0x7C00                           # bit patterns 1 .. 0x7BFF are the positive finite fp16
    bounds = [1]
    acc = 0
    for i in range(1, top):                # chunks of ~48M elements
        acc += 2 * i + 1
        if acc > 48_000_000:
            bounds.append(i + 1)
            acc = 0
    bounds.append(top)
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        x = _anchor_groups(lo, hi)
        int4_check(x, 128)
