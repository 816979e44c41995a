"""GPU parity of the appended-residual MXFP4 path against the oracle: the
two-pass quantizer's codes and scales bit for bit (including an exhaustive
sweep of fp16 inputs), the weight-side copy, and the unchanged block-scaled
GEMM over K' = 2K (block integers exact, Y within 1e-5 * T + 1e-6)."""
import numpy as np
import pytest

import oracle
from w4a4_quantized_gemm_quantize_amd import synth
from helpers import assert_y_close, dev, host

pytestmark = pytest.mark.gpu


def ops():
    from w4a4_quantized_gemm_quantize_amd import ops as o
    return o


def res_check(x16, ldx_pad=0, fn="mxfp4_quantize_residual"):
    R, K = x16.shape
    if ldx_pad:
        buf = np.zeros((R, K + ldx_pad), np.float16)
        buf[:, :K] = x16
        xt = dev(buf)[:, :K]
    else:
        xt = dev(x16)
    q, e = getattr(ops(), fn)(xt)
    if fn == "mxfp4_quantize_residual":
        codes, e8 = oracle.mxfp4_quantize_residual(x16)
    elif fn == "mxfp4_quantize_residual_tied":
        codes, e8 = oracle.mxfp4_quantize_residual_tied(x16)
    else:
        codes, e8 = oracle.mxfp4_append_copy(*oracle.mxfp4_quantize(x16))
    assert np.array_equal(oracle.from_panels(host(e), oracle.e8m0_panel_offsets(R, 2 * K)), e8), f"{fn} E8M0 (R={R} K={K})"
    bad = np.argwhere(host(q) != oracle.pack_nibbles(codes))
    assert bad.size == 0, f"{fn} codes differ at {bad[:5].tolist()} (R={R} K={K})"


@pytest.mark.parametrize("fn", ["mxfp4_quantize_residual", "mxfp4_quantize_append_copy",
                                "mxfp4_quantize_residual_tied"])
def test_shapes(fn):
    res_check(synth.activations(16, 256, dist="normal", seed=0), fn=fn)
    res_check(synth.activations(33, 3584, dist="t3", seed=5), ldx_pad=32, fn=fn)
    res_check(synth.activations(7, 1120, dist="t3", seed=9), fn=fn)     # last panel 3 blocks wide
    res_check(synth.activations(5, 96, dist="t3", seed=10), fn=fn)      # 2K = 192: panels of 6
    x = synth.activations(9, 512, dist="t3", seed=6)
    x[3] = 0
    x[4, :64] = np.float16(-0.0)
    res_check(x, fn=fn)
    res_check(synth.weights(40, 3584, seed=7), fn=fn)


def test_residual_exhaustive_fp16():
    """Every finite fp16 value in blocks with assorted absmax anchors: the
    first pass sees every input, the second pass the residuals they leave."""
    rng = np.random.default_rng(2)
    allf = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16)
    allv = np.concatenate([allf, -allf])
    perm = rng.permutation(allv)
    perm = np.concatenate([perm, np.zeros((-perm.size) % 31, np.float16)])
    blocks = perm.reshape(-1, 31)
    anchors = np.abs(blocks.astype(np.float32)).max(axis=1) * rng.choice([1, 1.25, 1.5, 3, 7, 1000], size=blocks.shape[0])
    anchors = np.clip(anchors, 0, 65504).astype(np.float16)
    x = np.concatenate([anchors[:, None], blocks], axis=1).reshape(-1)
    x = np.concatenate([x, np.zeros((-x.size) % 1024, np.float16)]).reshape(-1, 1024)
    res_check(x)


def gemm_case(M, N, K, seed=0, window=None):
    o = ops()
    x = synth.activations(M, K, dist="t3", seed=seed)
    w = synth.weights(N, K, seed=seed)
    xq, xe = o.mxfp4_quantize_residual(dev(x))
    wq, we = o.mxfp4_quantize_append_copy(dev(w))
    y = o.mxfp4_gemm(xq, xe, wq, we)
    ca, ea = oracle.mxfp4_quantize_residual(x)
    cw, ew = oracle.mxfp4_append_copy(*oracle.mxfp4_quantize(w))
    Y, T = oracle.mxfp4_gemm(ca, ea, cw, ew)
    assert_y_close(host(y), Y, T, f"appended mxfp4 M={M} N={N} K={K}")
    m0, mc, n0, nc = window if window else (0, M, 0, N)
    part = host(o.mxfp4_gemm_debug_partials(xq, xe, wq, we, m0, mc, n0, nc))
    for b, I in oracle.mxfp4_block_partials(ca[m0:m0 + mc], cw[n0:n0 + nc]):
        assert np.array_equal(part[b], I), f"block integers differ in block {b}"


@pytest.mark.parametrize("M,N,K", [(16, 256, 256), (130, 200, 512), (257, 129, 384), (64, 96, 1024)])
def test_appended_gemm(M, N, K):
    gemm_case(M, N, K, seed=M)


def test_qwen_w13_sampled():
    """Full-size Qwen2.5-7B w1 shape with the residual appended (K' = 7168),
    production launch configuration; checked on every column of 64 sampled rows."""
    o = ops()
    M, K, N = 4096, 3584, 18944
    x = synth.activations(M, K, dist="t3", seed=0)
    w = synth.weights(N, K, seed=0)
    xq, xe = o.mxfp4_quantize_residual(dev(x))
    wq, we = o.mxfp4_quantize_append_copy(dev(w))
    y = host(o.mxfp4_gemm(xq, xe, wq, we))
    rows = synth.sample_rows(M, 64, seed=2)
    ca, ea = oracle.mxfp4_quantize_residual(x[rows])
    cw, ew = oracle.mxfp4_append_copy(*oracle.mxfp4_quantize(w))
    Y, T = oracle.mxfp4_gemm(ca, ea, cw, ew)
    assert_y_close(y[rows], Y, T, "qwen w13 appended")


def test_qwen_w13_tied():
    """Full-size Qwen2.5-7B w1 shape with the tied residual appended (K' = 7168):
    every column of 64 sampled rows."""
    o = ops()
    M, K, N = 4096, 3584, 18944
    x = synth.activations(M, K, dist="t3", seed=1)
    w = synth.weights(N, K, seed=1)
    xq, xe = o.mxfp4_quantize_residual_tied(dev(x))
    wq, we = o.mxfp4_quantize_append_copy(dev(w))
    y = host(o.mxfp4_gemm(xq, xe, wq, we))
    rows = synth.sample_rows(M, 64, seed=4)
    ca, ea = oracle.mxfp4_quantize_residual_tied(x[rows])
    cw, ew = oracle.mxfp4_append_copy(*oracle.mxfp4_quantize(w))
    Y, T = oracle.mxfp4_gemm(ca, ea, cw, ew)
    assert_y_close(y[rows], Y, T, "qwen w13 tied")


def test_tied_every_value_under_every_first_exponent():
    """The tied two-pass quantizer bit for bit over every (x, E1) pair an fp16
    block can produce (the blocks of the oracle pin that proves the 1/64 bound)."""
    f16 = np.arange(1, 0x7C00, dtype=np.uint16)
    v = f16.view(np.float16).astype(np.float64)
    blocks = []
    for E1 in range(-25, 15):
        sel = (v <= 6 * 2.0 ** E1) & (v > 6 * 2.0 ** (E1 - 1))
        a = int(f16[sel].max())
        xs = np.concatenate([np.arange(0, a + 1, dtype=np.uint16),
                             np.arange(0, a + 1, dtype=np.uint16) | np.uint16(0x8000)])
        n = -(-xs.size // 31)
        pad = np.zeros(n * 31, np.uint16)
        pad[:xs.size] = xs
        b = np.empty((n, 32), np.uint16)
        b[:, 0] = a
        b[:, 1:] = pad.reshape(n, 31)
        blocks.append(b)
    x = np.concatenate(blocks)
    x = np.concatenate([x, np.zeros(((-x.shape[0]) % 32, 32), np.uint16)]).reshape(-1, 1024).view(np.float16)
    res_check(x, fn="mxfp4_quantize_residual_tied")


def test_tied_gemm():
    """The unchanged block-scaled GEMM over the tied activation side and the
    appended weight copy: Y within the oracle bound."""
    M, N, K = 130, 200, 768
    x = synth.activations(M, K, dist="t3", seed=12)
    w = synth.weights(N, K, seed=13)
    q, e = ops().mxfp4_quantize_residual_tied(dev(x))
    wq, we = ops().mxfp4_quantize_append_copy(dev(w))
    y = host(ops().mxfp4_gemm(q, e, wq, we))
    ca, ea = oracle.mxfp4_quantize_residual_tied(x)
    cw, ew = oracle.mxfp4_append_copy(*oracle.mxfp4_quantize(w))
    Y, T = oracle.mxfp4_gemm(ca, ea, cw, ew)
    assert_y_close(y, Y, T, "tied two-pass GEMM")
