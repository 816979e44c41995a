"""GPU parity of the storage conversions (canonical <-> GEMM layouts), and
"drop-in" use: codes and scales packed canonically by the oracle's layout
module (two's-complement INT4 nibbles, row-major scales) go through the
conversion calls into the GEMMs, whose outputs must match the oracle."""
import numpy as np
import pytest

import oracle
from w4a4_quantized_gemm_quantize_amd import synth
from helpers import assert_y_close, dev, host

pytestmark = pytest.mark.gpu


def ops():
    from w4a4_quantized_gemm_quantize_amd import ops as o
    return o


@pytest.mark.parametrize("R,K", [(1, 16), (37, 512), (300, 1024)])
def test_repack_and_unpack_int4(R, K):
    x = synth.activations(R, K, seed=R + K)
    codes, _ = oracle.int4_quantize(x, 16 if K == 16 else 128)
    packed, count = ops().w4a4_repack_int4(dev(oracle.pack_int4_twos(codes)))
    assert host(count)[0] == 0
    assert np.array_equal(host(packed), oracle.pack_int4(codes, codes < 0)), "canonical -> GEMM layout"
    # the library's own quantizer output (with -0 codes) back to canonical form
    xq, _ = ops().w4a4_quantize_act(dev(x), 16 if K == 16 else 128)
    assert np.array_equal(host(ops().w4a4_unpack_int4(xq)), oracle.pack_int4_twos(codes)), "GEMM -> canonical"


def test_repack_counts_minus_eight():
    rng = np.random.default_rng(5)
    codes = rng.integers(-8, 8, size=(64, 256)).astype(np.int8)
    n8 = int((codes == -8).sum())
    assert n8 > 0
    packed, count = ops().w4a4_repack_int4(dev(oracle.pack_int4_twos(codes)), check=False)
    assert host(count)[0] == n8
    zeroed = np.where(codes == -8, 0, codes)
    assert np.array_equal(host(packed), oracle.pack_int4(zeroed, zeroed < 0)), "-8 codes are stored as 0"
    with pytest.raises(ValueError):
        ops().w4a4_repack_int4(dev(oracle.pack_int4_twos(codes)))
    # a second call clears the count first
    ok = np.where(codes == -8, 3, codes)
    _, count2 = ops().w4a4_repack_int4(dev(oracle.pack_int4_twos(ok)))
    assert host(count2)[0] == 0


@pytest.mark.parametrize("rows,groups", [(1, 1), (33, 7), (1000, 64), (4096, 1)])
def test_scale_transposes(rows, groups):
    s = np.random.default_rng(rows).random((rows, groups), dtype=np.float32)
    gm = ops().w4a4_scales_to_group_major(dev(s))
    assert np.array_equal(host(gm), s.T)
    assert np.array_equal(host(ops().w4a4_scales_to_row_major(gm)), s)


@pytest.mark.parametrize("M,N,K,ga,gw", [(300, 392, 1024, 128, 128), (65, 130, 512, 64, 128), (257, 96, 768, 768, 128)])
def test_int4_drop_in(M, N, K, ga, gw):
    """Canonical INT4 data packed by the oracle -> conversions -> w4a4_gemm."""
    o = ops()
    qa, sa = oracle.int4_quantize(synth.activations(M, K, seed=M), ga)
    qw, sw = oracle.int4_quantize(synth.weights(N, K, seed=N), gw)
    xq, _ = o.w4a4_repack_int4(dev(oracle.pack_int4_twos(qa)))
    wq, _ = o.w4a4_repack_int4(dev(oracle.pack_int4_twos(qw)))
    xs = o.w4a4_scales_to_group_major(dev(sa))
    ws = o.w4a4_scales_to_group_major(dev(sw))
    Y, T = oracle.w4a4_gemm(qa, sa, ga, qw, sw, gw)
    assert_y_close(host(o.w4a4_gemm(xq, xs, ga, wq, ws, gw)), Y, T, "drop-in INT4")
    part = host(o.w4a4_gemm_debug_partials(xq, xs, ga, wq, ws, gw, 0, M, 0, N))
    for b, P in oracle.w4a4_block_partials(qa, qw, min(ga, gw)):
        assert np.array_equal(part[b], P), f"drop-in partials block {b}"


@pytest.mark.parametrize("M,N,K", [(200, 160, 1024), (64, 256, 384)])
def test_mxfp4_drop_in(M, N, K):
    o = ops()
    ca, ea = oracle.mxfp4_quantize(synth.activations(M, K, seed=K))
    cw, ew = oracle.mxfp4_quantize(synth.weights(N, K, seed=M))
    xe = o.mxfp4_scales_to_panels(dev(ea))
    we = o.mxfp4_scales_to_panels(dev(ew))
    assert np.array_equal(host(xe), oracle.to_panels(ea, oracle.e8m0_panel_offsets(M, K)))
    assert np.array_equal(host(o.mxfp4_scales_to_rows(xe, M, K)), ea)
    y = o.mxfp4_gemm(dev(oracle.pack_nibbles(ca)), xe, dev(oracle.pack_nibbles(cw)), we)
    Y, T = oracle.mxfp4_gemm(ca, ea, cw, ew)
    assert_y_close(host(y), Y, T, "drop-in MXFP4")


def test_nvfp4_drop_in():
    import torch
    o = ops()
    M, N, K = 130, 200, 512
    x = synth.activations(M, K, seed=1)
    w = synth.weights(N, K, seed=2)
    gx, gw = oracle.nvfp4_global_scale(x), oracle.nvfp4_global_scale(w)
    cx, sx = oracle.nvfp4_quantize(x, gx)
    cw, sw = oracle.nvfp4_quantize(w, gw)
    xs = o.nvfp4_scales_to_panels(dev(sx))
    ws = o.nvfp4_scales_to_panels(dev(sw))
    assert np.array_equal(host(o.nvfp4_scales_to_rows(xs, M, K)), sx)
    gxt = torch.tensor([gx], dtype=torch.float32, device="cuda")
    gwt = torch.tensor([gw], dtype=torch.float32, device="cuda")
    y = o.nvfp4_gemm(dev(oracle.pack_nibbles(cx)), xs, gxt, dev(oracle.pack_nibbles(cw)), ws, gwt)
    Y, T = oracle.nvfp4_gemm(cx, sx, gx, cw, sw, gw)
    assert_y_close(host(y), Y, T, "drop-in NVFP4")
