"""GPU parity of the NVFP4 path against the oracle.

Global scale, E4M3 block scales and E2M1 codes are integer decisions: they must
match the oracle bit for bit (the kernel and the oracle take them in the same
binary32 arithmetic). The GEMM's per-block integers I_b = sum (2vx)(2vw) come
from the debug entry point (same loads and fp16 conversion, unit scales) and
must match exactly; Y must satisfy |Y_gpu - Y| <= 1e-5 * T + 1e-6 with
T = g_x g_w sum_b |s_x s_w I_b / 4|, and is bit-exact on inputs whose every
partial sum is representable."""
import numpy as np
import pytest

import oracle
from w4a4_quantized_gemm_quantize_amd import synth
from helpers import assert_y16_close, assert_y_close, dev, host

pytestmark = pytest.mark.gpu


def ops():
    from w4a4_quantized_gemm_quantize_amd import ops as o
    return o


def gdev(v):
    return dev(np.array([v], np.float32))


# ------------------------------------------------------------- quantizer
def nv_check(x16, sg=None, ldx_pad=0, what=""):
    """Quantize on the GPU and compare codes and scale bytes with the oracle.
    sg=None: the global scale comes from the device kernel and must equal the
    oracle's."""
    R, K = x16.shape
    if ldx_pad:
        buf = np.zeros((R, K + ldx_pad), np.float16)
        buf[:, :K] = x16
        xt = dev(buf)[:, :K]
    else:
        xt = dev(x16)
    if sg is None:
        g = ops().nvfp4_global_scale(xt)
        sg = oracle.nvfp4_global_scale(x16)
        assert host(g).view(np.uint32)[0] == np.float32(sg).view(np.uint32), f"global scale {what}"
    else:
        g = gdev(sg)
    q, s = ops().nvfp4_quantize(xt, g)
    codes, sb = oracle.nvfp4_quantize(x16, sg)
    got_s = oracle.from_panels(host(s), oracle.e4m3_panel_offsets(R, K))
    bad = np.argwhere(got_s != sb)
    assert bad.size == 0, f"E4M3 scales differ at {bad[:5].tolist()} {what}"
    gq = host(q)
    want = oracle.pack_nibbles(codes)
    bad = np.argwhere(gq != want)
    assert bad.size == 0, f"codes differ at {bad[:5].tolist()} {what}"


def test_global_scale():
    for seed, (R, K) in enumerate([(1, 8), (3, 256), (130, 3584), (4096, 256)]):
        x = synth.activations(R, K, dist="t3", seed=seed)
        g = ops().nvfp4_global_scale(dev(x))
        assert host(g)[0] == oracle.nvfp4_global_scale(x), (R, K)
    x = np.zeros((5, 64), np.float16)
    x[4, 63] = -60000.0                           # the absmax is negative
    assert host(ops().nvfp4_global_scale(dev(x)))[0] == oracle.nvfp4_global_scale(x)
    assert host(ops().nvfp4_global_scale(dev(np.zeros((3, 16), np.float16))))[0] == 0.0
    g = gdev(7.0)
    ops().nvfp4_global_scale(dev(np.zeros((0, 16), np.float16)), out=g)
    assert host(g)[0] == 0.0


def test_quantize_shapes():
    nv_check(synth.activations(16, 256, dist="normal", seed=0), what="tiny")
    nv_check(synth.activations(33, 3584, dist="t3", seed=5), ldx_pad=32, what="strided")
    x = synth.activations(7, 18944, dist="t3", seed=6)
    x[3, :64] = 0
    nv_check(x, what="long rows")
    nv_check(synth.weights(40, 3584, seed=7), what="weights")
    nv_check(synth.activations(1, 256, dist="t3", seed=9), what="one row")
    nv_check(synth.activations(257, 768, dist="t3", seed=10), what="ragged rows")


def test_quantize_given_global_scales():
    x = synth.activations(24, 512, dist="t3", seed=3)
    amax = float(np.abs(x.astype(np.float32)).max())
    for sg in (amax / 2688, amax / 2688 * 1.37, amax / 2688 / 50,   # block scales saturating at 448
               amax / 2688 * 1e4, 2.0 ** -20, 0.0):                 # tiny / zero block scales
        nv_check(x, sg=np.float32(sg), what=f"sg={sg}")


def test_quantize_edge_values():
    x = np.zeros((4, 256), np.float16)
    x[0, 16] = 3.0
    x[0, 17] = np.float16(-1e-4)      # magnitude rounds to 0: sign bit kept
    x[0, 18] = np.float16(-0.0)
    x[1, :16] = np.float16(2.0 ** -24)  # smallest fp16 subnormal
    x[2, 32:48] = np.linspace(-6, 6, 16).astype(np.float16)
    x[3] = synth.activations(1, 256, dist="t3", seed=2)[0]
    nv_check(x, what="edges")
    nv_check(x, sg=np.float32(1.0), what="edges sg=1")
    nv_check(x, sg=np.float32(0.25), what="edges sg=1/4")


def test_quantize_scale_ties():
    """Block absmax values whose r = a / d lands on E4M3 rounding midpoints."""
    grid = oracle.e4m3_decode(np.arange(1, 0x7F))
    mids = (grid[:-1] + grid[1:]) / 2
    rows = []
    for m in mids:
        blk = np.zeros(16, np.float64)
        blk[3] = m * 6.0 * 2.0 ** -4          # s_g = 2^-4: d = 6/16, a = m d exactly if representable
        blk[7] = -0.3 * blk[3]
        rows.append(blk)
    flat = np.concatenate(rows)
    flat = np.concatenate([flat, np.zeros((-flat.size) % 256)])
    x = flat.reshape(-1, 256).astype(np.float16)
    nv_check(x, sg=np.float32(2.0 ** -4), what="E4M3 ties")


def test_quantize_exhaustive_fp16():
    """Every finite fp16 value, in blocks [anchor, 15 values], over four
    magnitude bands each quantized with its own global scale."""
    rng = np.random.default_rng(1)
    allf = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16)
    allv = np.concatenate([allf, -allf])
    order = np.argsort(np.abs(allv.astype(np.float32)), kind="stable")
    for band in np.array_split(allv[order], 4):
        perm = rng.permutation(band)
        perm = np.concatenate([perm, np.zeros((-perm.size) % 15, np.float16)])
        blocks = perm.reshape(-1, 15)
        anchors = np.abs(blocks.astype(np.float32)).max(axis=1) * rng.choice([1, 1.5, 3, 7], size=blocks.shape[0])
        anchors = np.clip(anchors, 0, 65504).astype(np.float16)
        x = np.concatenate([anchors[:, None], blocks], axis=1).reshape(-1)
        x = np.concatenate([x, np.zeros((-x.size) % 1024, np.float16)]).reshape(-1, 1024)
        nv_check(x, what="exhaustive band")


def _every_scale_blocks(sg):
    """Blocks [a_b, x_1..x_15] where a_b = fp16(fl32(6 s_g) * E4M3 value b) for
    every E4M3 byte b = 1..126 (so the block gets scale byte b: the fp16
    rounding of a_b is far finer than E4M3 spacing) and the x run over every
    fp16 value with |x| <= a_b, both signs; zero-padded to rows of 256."""
    d = np.float32(np.float32(6) * np.float32(sg))
    vals = oracle.e4m3_decode(np.arange(1, 0x7F))
    pos = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
    blocks = []
    for v in vals:
        a = np.float16(d * np.float32(v))
        if not np.isfinite(a) or a == 0:
            continue
        xs = pos[pos <= np.float32(a)]
        xs = np.concatenate([xs, -xs[1:]]).astype(np.float16)
        n = -(-xs.size // 15)
        pad = np.zeros(n * 15, np.float16)
        pad[:xs.size] = xs
        blk = np.empty((n, 16), np.float16)
        blk[:, 0] = a
        blk[:, 1:] = pad.reshape(n, 15)
        blocks.append(blk)
    flat = np.concatenate(blocks).reshape(-1)
    flat = np.concatenate([flat, np.zeros((-flat.size) % 256, np.float16)])
    return flat.reshape(-1, 256)


@pytest.mark.parametrize("sg", [2.0 ** -4, 0.37])
def test_quantize_every_scale_every_x(sg):
    """Every reachable block scale (126 E4M3 bytes for this global scale) with
    every fp16 input at or below its block's absmax: every code decision the
    quantizer can take under that global scale, bit-exact."""
    x = _every_scale_blocks(sg)
    nv_check(x, sg=np.float32(sg), what=f"every scale x every x, sg={sg}")


# ------------------------------------------------------------------ GEMM
def run_case(M, N, K, seed=0, window=None, dist="t3", check_fp16=False):
    import torch
    o = ops()
    x = synth.activations(M, K, dist=dist, seed=seed)
    w = synth.weights(N, K, seed=seed)
    xt, wt = dev(x), dev(w)
    gx, gw = o.nvfp4_global_scale(xt), o.nvfp4_global_scale(wt)
    xq, xs = o.nvfp4_quantize(xt, gx)
    wq, ws = o.nvfp4_quantize(wt, gw)
    y = o.nvfp4_gemm(xq, xs, gx, wq, ws, gw)
    sgx, sgw = oracle.nvfp4_global_scale(x), oracle.nvfp4_global_scale(w)
    ca, sa = oracle.nvfp4_quantize(x, sgx)
    cw, sw = oracle.nvfp4_quantize(w, sgw)
    Y, T = oracle.nvfp4_gemm(ca, sa, sgx, cw, sw, sgw)
    ratio = assert_y_close(host(y), Y, T, f"nvfp4 M={M} N={N} K={K}")
    if check_fp16:
        y16 = o.nvfp4_gemm(xq, xs, gx, wq, ws, gw, out_dtype=torch.float16)
        assert_y16_close(host(y16).astype(np.float64), Y, T, "nvfp4 fp16")
    m0, mc, n0, nc = window if window else (0, M, 0, N)
    part = host(o.nvfp4_gemm_debug_partials(xq, xs, wq, ws, m0, mc, n0, nc))
    for b, I in oracle.nvfp4_block_partials(ca[m0:m0 + mc], cw[n0:n0 + nc]):
        assert np.array_equal(part[b], I), f"block integers differ in block {b}"
    return ratio


def test_tiny():
    run_case(16, 256, 256, dist="normal", check_fp16=True)


@pytest.mark.parametrize("M,N,K", [(1, 128, 256), (130, 200, 512), (300, 392, 1024), (257, 129, 768),
                                   (513, 520, 256)])
def test_ragged_shapes(M, N, K):
    run_case(M, N, K, seed=M, check_fp16=(M == 130))


def test_exact_regime_bit_exact():
    """Power-of-two block scales (every 16-block's absmax 6 * 2^e, e in
    {-1, 0, 1}) and s_g = 1: every product and partial sum is a multiple of
    2^-4 below 2^20, so Y is exact in fp32 whatever the summation order."""
    rng = np.random.default_rng(5)
    M, N, K = 96, 160, 1024

    def mat(R):
        v = oracle.e2m1_decode(rng.integers(0, 16, (R, K)))
        e = rng.integers(-1, 2, (R, K // 16))
        v = v.reshape(R, K // 16, 16)
        v[:, :, 0] = 6.0
        return (v * np.exp2(e)[:, :, None]).reshape(R, K).astype(np.float16)

    x, w = mat(M), mat(N)
    o = ops()
    one = gdev(1.0)
    xq, xs = o.nvfp4_quantize(dev(x), one)
    wq, ws = o.nvfp4_quantize(dev(w), one)
    y = host(o.nvfp4_gemm(xq, xs, one, wq, ws, one))
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.array_equal(y.astype(np.float64), ref)


def test_zero_rows_and_blocks():
    M, N, K = 48, 64, 512
    o = ops()
    x = synth.activations(M, K, seed=2)
    x[:, 64:128] = 0
    x[5] = 0
    w = synth.weights(N, K, seed=2)
    gx, gw = o.nvfp4_global_scale(dev(x)), o.nvfp4_global_scale(dev(w))
    xq, xs = o.nvfp4_quantize(dev(x), gx)
    wq, ws = o.nvfp4_quantize(dev(w), gw)
    y = host(o.nvfp4_gemm(xq, xs, gx, wq, ws, gw))
    sgx, sgw = oracle.nvfp4_global_scale(x), oracle.nvfp4_global_scale(w)
    Y, T = oracle.nvfp4_gemm(*oracle.nvfp4_quantize(x, sgx), sgx, *oracle.nvfp4_quantize(w, sgw), sgw)
    assert_y_close(y, Y, T, "zero blocks")
    assert np.all(y[5] == 0)


def test_full_row_tiles_fp16_and_strided_y():
    import torch
    M, N, K = 512, 200, 512
    run_case(M, N, K, seed=7, check_fp16=True)
    o = ops()
    x = synth.activations(M, K, seed=8)
    w = synth.weights(N, K, seed=8)
    gx, gw = o.nvfp4_global_scale(dev(x)), o.nvfp4_global_scale(dev(w))
    xq, xs = o.nvfp4_quantize(dev(x), gx)
    wq, ws = o.nvfp4_quantize(dev(w), gw)
    sgx, sgw = oracle.nvfp4_global_scale(x), oracle.nvfp4_global_scale(w)
    Y, T = oracle.nvfp4_gemm(*oracle.nvfp4_quantize(x, sgx), sgx, *oracle.nvfp4_quantize(w, sgw), sgw)
    for dt in (torch.float32, torch.float16):
        big = torch.full((M, N + 40), 7.0, dtype=dt, device="cuda")
        o.nvfp4_gemm(xq, xs, gx, wq, ws, gw, out_dtype=dt, out=big[:, :N])
        b = host(big).astype(np.float64)
        assert np.all(b[:, N:] == 7.0), "padding columns written"
        if dt == torch.float32:
            assert_y_close(b[:, :N], Y, T, "strided fp32")
        else:
            assert_y16_close(b[:, :N], Y, T, "strided fp16")


def test_empty_is_noop():
    import torch
    o = ops()
    xq = torch.zeros((0, 128), dtype=torch.uint8, device="cuda")
    xs = torch.zeros((0,), dtype=torch.uint8, device="cuda")
    wq = torch.zeros((8, 128), dtype=torch.uint8, device="cuda")
    ws = torch.zeros((8 * 16,), dtype=torch.uint8, device="cuda")
    one = gdev(1.0)
    y = o.nvfp4_gemm(xq, xs, one, wq, ws, one)
    assert y.shape == (0, 8)


@pytest.mark.parametrize("name", ["qwen25_7b_w13", "qwen25_7b_w2"])
def test_qwen_shapes_sampled(name):
    """The production launch at the Qwen2.5-7B FFN shapes, checked on every
    column of a seeded sample of 64 rows, and bit-exact block integers in a
    window."""
    wl = synth.WORKLOADS[name]
    M, N, K = wl["M"], wl["N"], wl["K"]
    o = ops()
    x = synth.activations(M, K, dist="t3", seed=0)
    w = synth.weights(N, K, seed=0)
    xt, wt = dev(x), dev(w)
    gx, gw = o.nvfp4_global_scale(xt), o.nvfp4_global_scale(wt)
    xq, xs = o.nvfp4_quantize(xt, gx)
    wq, ws = o.nvfp4_quantize(wt, gw)
    sgx, sgw = oracle.nvfp4_global_scale(x), oracle.nvfp4_global_scale(w)
    del wt, xt
    y = host(o.nvfp4_gemm(xq, xs, gx, wq, ws, gw))
    rows = synth.sample_rows(M, 64, seed=2)
    ca, sa = oracle.nvfp4_quantize(x[rows], sgx)
    cw, sw = oracle.nvfp4_quantize(w, sgw)
    Y, T = oracle.nvfp4_gemm(ca, sa, sgx, cw, sw, sgw)
    assert_y_close(y[rows], Y, T, name)
    m0, n0, win = M // 2 - 8, N // 2 - 8, 16
    part = host(o.nvfp4_gemm_debug_partials(xq, xs, wq, ws, m0, win, n0, win))
    ca2, _ = oracle.nvfp4_quantize(x[m0:m0 + win], sgx)
    cw2, _ = oracle.nvfp4_quantize(w[n0:n0 + win], sgw)
    for b, I in oracle.nvfp4_block_partials(ca2, cw2):
        assert np.array_equal(part[b], I), f"block {b}"
