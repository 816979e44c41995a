"""w4a4_gemm_splitk_noalloc (the entry point for callers that cannot
allocate: split partials in the library's static device buffer) against
w4a4_gemm_splitk with a caller workspace, through the C ABI: two calls in a
row, the second smaller, each bit-identical to the workspace variant (same
kernels, same split plan, same fixed-order reduction) and within the oracle's
bound on sampled outputs."""
import numpy as np
import pytest

import oracle
from w4a4_quantized_gemm_quantize_amd import _lib, synth
from helpers import assert_y_close, dev, host

pytestmark = pytest.mark.gpu


def _call_noalloc(xq, xs, ga, wq, ws, gw, M, N, K, y, splits=0):
    import torch
    _lib.call("w4a4_gemm_splitk_noalloc", xq.data_ptr(), xs.data_ptr(), ga, wq.data_ptr(), ws.data_ptr(), gw,
              M, N, K, splits, y.data_ptr(), _lib.Y_F32, y.stride(0), torch.cuda.current_stream().cuda_stream)


def _case(M, N, K, seed):
    import torch
    from w4a4_quantized_gemm_quantize_amd import ops
    x = synth.activations(M, K, seed=seed)
    w = synth.weights(N, K, seed=seed + 1)
    xq, xs = ops.w4a4_quantize_act(dev(x), 128)
    wq, ws = ops.w4a4_pack_weight(dev(w), 128)
    assert _lib.splitk_workspace_bytes(M, N, K, 128, 128, 0) > 0, "the shape must split"
    y_ref = ops.w4a4_gemm_splitk(xq, xs, 128, wq, ws, 128)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    _call_noalloc(xq, xs, 128, wq, ws, 128, M, N, K, y)
    yh = host(y)
    assert np.array_equal(yh, host(y_ref)), f"noalloc differs from the workspace call (M={M} N={N} K={K})"
    rows = synth.sample_rows(M, 6, seed=seed)
    cols = synth.sample_rows(N, 200, seed=seed)
    qa, sa = oracle.int4_quantize(x[rows], 128)
    qw, sw = oracle.int4_quantize(w[cols], 128)
    Y, T = oracle.w4a4_gemm(qa, sa, 128, qw, sw, 128)
    assert_y_close(yh[np.ix_(rows, cols)], Y, T, f"noalloc M={M} N={N} K={K}")


def test_noalloc_matches_workspace_call_twice():
    # first the largest plan the buffer holds (LLaMA-2-70B w2 at 256 tokens:
    # 4 splits x 256 x 8192 fp32 = 32 MiB), then a smaller one
    assert _lib.load_library().w4a4_gemm_splitk_noalloc_max_bytes() == 32 << 20
    assert _lib.splitk_workspace_bytes(256, 8192, 28672, 128, 128, 0) == 32 << 20
    _case(256, 8192, 28672, seed=3)
    _case(100, 1000, 2048, seed=4)


def test_noalloc_rejects_plans_beyond_the_buffer():
    import torch
    from w4a4_quantized_gemm_quantize_amd import ops
    M, N, K = 512, 8192, 4096                     # 8 splits x 512 x 8192 x 4 B = 128 MiB
    xq = torch.zeros((M, K // 2), dtype=torch.uint8, device="cuda")
    xs = torch.zeros((K // 128, M), dtype=torch.float32, device="cuda")
    wq = torch.zeros((N, K // 2), dtype=torch.uint8, device="cuda")
    ws = torch.zeros((K // 128, N), dtype=torch.float32, device="cuda")
    y = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    st = _lib.status_of("w4a4_gemm_splitk_noalloc", xq.data_ptr(), xs.data_ptr(), 128, wq.data_ptr(),
                        ws.data_ptr(), 128, M, N, K, 8, y.data_ptr(), 0, N, None)
    assert st == 7                               # W4A4_E_SCRATCH, nothing launched
    torch.cuda.synchronize()
    assert float(y.abs().max()) == 0.0
    del ops
