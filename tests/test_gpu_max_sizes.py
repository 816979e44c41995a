"""GPU parity at the longest reduction the GEMMs accept, K = 2^23 (the cap
that keeps a 256-row tile's byte offsets in 32 bits): the tiled INT4 kernel
on 256-row tiles, its automatic K split, the few-token path, and the MXFP4
kernel, each checked against the oracle on sampled outputs; the INT4
partials bit-exact in a window (65536 groups per output)."""
import numpy as np
import pytest

import oracle
from w4a4_quantized_gemm_quantize_amd import synth
from helpers import assert_y_close, dev, host

pytestmark = pytest.mark.gpu

KMAX = 1 << 23
M, N = 136, 40          # > 128 rows: 256-row tiles; N ragged against 128-column tiles


@pytest.fixture(scope="module")
def data():
    x = synth.bulk_normal(M, KMAX, seed=21)                          # ~2.3 GB of fp16
    w = (synth.bulk_normal(N, KMAX, seed=22).astype(np.float32) * 0.02).astype(np.float16)
    rows = synth.sample_rows(M, 6, seed=23)
    cols = synth.sample_rows(N, 8, seed=24)
    yield x, w, rows, cols


def ops():
    from w4a4_quantized_gemm_quantize_amd import ops as o
    return o


def test_int4_longest_k(data):
    x, w, rows, cols = data
    o = ops()
    print(f"int4 M={M} N={N} K={KMAX}", flush=True)
    xq, xs = o.w4a4_quantize_act(dev(x), 128)
    wq, ws = o.w4a4_pack_weight(dev(w), 128)
    y = host(o.w4a4_gemm(xq, xs, 128, wq, ws, 128))
    y_split = host(o.w4a4_gemm_splitk(xq, xs, 128, wq, ws, 128))
    qa, sa = oracle.int4_quantize(x[rows], 128)
    qw, sw = oracle.int4_quantize(w[cols], 128)
    Y, T = oracle.w4a4_gemm(qa, sa, 128, qw, sw, 128)
    assert_y_close(y[np.ix_(rows, cols)], Y, T, "tiled, K = 2^23")
    assert_y_close(y_split[np.ix_(rows, cols)], Y, T, "split K, K = 2^23")
    # partials of a 4 x 4 window across the last rows and columns
    m0, n0 = M - 4, N - 4
    part = host(o.w4a4_gemm_debug_partials(xq, xs, 128, wq, ws, 128, m0, 4, n0, 4))
    qa2, _ = oracle.int4_quantize(x[m0:], 128)
    qw2, _ = oracle.int4_quantize(w[n0:], 128)
    nblk = 0
    for b, P in oracle.w4a4_block_partials(qa2, qw2, 128):
        assert np.array_equal(part[b], P), f"partials block {b}"
        nblk += 1
    assert nblk == KMAX // 128


def test_int4_few_tokens_longest_k(data):
    x, w, _, cols = data
    o = ops()
    print(f"int4 few tokens M=8 N={N} K={KMAX}", flush=True)
    xq, xs = o.w4a4_quantize_act(dev(x[:8]), 128)
    wq, ws = o.w4a4_pack_weight(dev(w), 128)
    y = host(o.w4a4_gemm(xq, xs, 128, wq, ws, 128))
    qa, sa = oracle.int4_quantize(x[:8], 128)
    qw, sw = oracle.int4_quantize(w[cols], 128)
    Y, T = oracle.w4a4_gemm(qa, sa, 128, qw, sw, 128)
    assert_y_close(y[:, cols], Y, T, "few-token path, K = 2^23")


def test_mxfp4_longest_k(data):
    x, w, rows, cols = data
    o = ops()
    print(f"mxfp4 M={M} N={N} K={KMAX}", flush=True)
    xq, xe = o.mxfp4_quantize(dev(x))
    wq, we = o.mxfp4_quantize(dev(w))
    y = host(o.mxfp4_gemm(xq, xe, wq, we))
    ca, ea = oracle.mxfp4_quantize(x[rows])
    cw, ew = oracle.mxfp4_quantize(w[cols])
    Y, T = oracle.mxfp4_gemm(ca, ea, cw, ew)
    assert_y_close(y[np.ix_(rows, cols)], Y, T, "MXFP4, K = 2^23")


def test_nvfp4_longest_k(data):
    x, w, rows, cols = data
    o = ops()
    print(f"nvfp4 M={M} N={N} K={KMAX}", flush=True)
    xt, wt = dev(x), dev(w)
    gx, gw = o.nvfp4_global_scale(xt), o.nvfp4_global_scale(wt)
    xq, xs = o.nvfp4_quantize(xt, gx)
    wq, ws = o.nvfp4_quantize(wt, gw)
    del xt, wt
    y = host(o.nvfp4_gemm(xq, xs, gx, wq, ws, gw))
    sgx, sgw = oracle.nvfp4_global_scale(x), oracle.nvfp4_global_scale(w)
    assert host(gx).view(np.uint32)[0] == np.float32(sgx).view(np.uint32), "global scale of X"
    ca, sa = oracle.nvfp4_quantize(x[rows], sgx)
    cw, sw = oracle.nvfp4_quantize(w[cols], sgw)
    Y, T = oracle.nvfp4_gemm(ca, sa, sgx, cw, sw, sgw)
    assert_y_close(y[np.ix_(rows, cols)], Y, T, "NVFP4, K = 2^23")
