"""GPU parity of the fused decode path (w4a4_linear_fused: activation
quantization inside the few-token GEMM, one launch). Its output must be
bit-identical to w4a4_quantize_act followed by w4a4_gemm (same quantizer
arithmetic, same wave split and fixed-order sums) and within the oracle's
bound; the full-size LLaMA-2-70B and 7B decode shapes (up to the largest M
whose LDS copy of X fits) are checked on every output."""
import numpy as np
import pytest

import oracle
from w4a4_quantized_gemm_quantize_amd import synth
from helpers import assert_y16_close, assert_y_close, dev, host

pytestmark = pytest.mark.gpu


def ops():
    from w4a4_quantized_gemm_quantize_amd import ops as o
    return o


def two_launch(o, xt, wq, ws, ga, gw, dtype=None):
    import torch
    xq, xs = o.w4a4_quantize_act(xt, ga)
    return o.w4a4_gemm(xq, xs, ga, wq, ws, gw, out_dtype=dtype or torch.float32)


@pytest.mark.parametrize("M,N,K,ga,gw", [
    (1, 200, 1024, 128, 128), (3, 96, 512, 64, 128), (7, 130, 1024, 256, 128),
    (2, 64, 1024, 512, 128), (5, 600, 768, 128, 256), (1, 16400, 256, 128, 128),   # 513 tiles: four waves
    (32, 40, 384, 128, 128), (4, 33, 2048, 64, 64)])
def test_fused_matches_two_launches_and_oracle(M, N, K, ga, gw):
    import torch
    o = ops()
    x = synth.activations(M, K, seed=M + N)
    w = synth.weights(N, K, seed=K)
    xt = dev(x)
    wq, ws = o.w4a4_pack_weight(dev(w), gw)
    y = host(o.w4a4_linear(xt, wq, ws, ga, gw, fused=True))
    assert np.array_equal(y, host(two_launch(o, xt, wq, ws, ga, gw))), "fused differs from quantize + gemm"
    Y, T = oracle.w4a4_gemm(*oracle.int4_quantize(x, ga), ga, *oracle.int4_quantize(w, gw), gw)
    assert_y_close(y, Y, T, f"fused M={M} N={N} K={K}")
    y16 = o.w4a4_linear(xt, wq, ws, ga, gw, out_dtype=torch.float16, fused=True)
    assert_y16_close(host(y16).astype(np.float64), Y, T, "fused fp16")


def test_fused_strided_x_and_y():
    import torch
    o = ops()
    M, N, K = 3, 72, 512
    x = synth.activations(M, K, seed=9)
    buf = np.zeros((M, K + 40), np.float16)
    buf[:, :K] = x
    xt = dev(buf)[:, :K]
    wq, ws = o.w4a4_pack_weight(dev(synth.weights(N, K, seed=9)), 128)
    big = torch.full((M, N + 8), 7.0, dtype=torch.float32, device="cuda")
    o.w4a4_linear(xt, wq, ws, 128, 128, out=big[:, :N], fused=True)
    b = host(big)
    assert np.all(b[:, N:] == 7.0)
    assert np.array_equal(b[:, :N], host(two_launch(o, dev(x), wq, ws, 128, 128)))


def test_fused_zero_rows_and_unsupported():
    o = ops()
    x = np.zeros((2, 256), np.float16)
    x[1, 100] = 3.0
    wq, ws = o.w4a4_pack_weight(dev(synth.weights(64, 256, seed=1)), 128)
    y = host(o.w4a4_linear(dev(x), wq, ws, 128, 128, fused=True))
    assert np.all(y[0] == 0)
    assert np.array_equal(y, host(two_launch(o, dev(x), wq, ws, 128, 128)))
    with pytest.raises(ValueError):       # 33 rows: beyond one row tile
        o.w4a4_linear(dev(np.zeros((33, 256), np.float16)), wq, ws, 128, 128, fused=True)
    wq1, ws1 = o.w4a4_pack_weight(dev(synth.weights(64, 1024, seed=2)), 128)
    with pytest.raises(ValueError):       # per-token activation groups are not fused
        o.w4a4_linear(dev(np.zeros((2, 1024), np.float16)), wq1, ws1, 1024, 128, fused=True)


@pytest.mark.parametrize("M,N,K", [(1, 28672, 8192), (8, 28672, 8192), (9, 28672, 8192), (1, 8192, 28672),
                                   (2, 8192, 28672), (7, 11008, 4096), (4, 4096, 11008)])   # last two: LLaMA-2-7B
def test_fused_llama_decode(M, N, K):
    o = ops()
    x = synth.activations(M, K, dist="t3", seed=0)
    w = synth.weights(N, K, seed=0)
    wq, ws = o.w4a4_pack_weight(dev(w), 128)
    xt = dev(x)
    y = host(o.w4a4_linear(xt, wq, ws, 128, 128, fused=True))
    assert np.array_equal(y, host(two_launch(o, xt, wq, ws, 128, 128))), "fused differs from quantize + gemm"
    Y, T = oracle.w4a4_gemm(*oracle.int4_quantize(x, 128), 128, *oracle.int4_quantize(w, 128), 128)
    assert_y_close(y, Y, T, f"fused decode M={M} N={N} K={K}")
