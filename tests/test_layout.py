"""Host-side layout helpers of the binding (CPU only): the 256-k panel layout
of MXFP4 scale bytes, checked against a loop written from the C header's
definition (panel p = blocks 8p.., rows of min(8, blocks left) bytes, the even
blocks' bytes before the odd ones')."""
import numpy as np
import pytest

from w4a4_quantized_gemm_quantize_amd import ops


def panels_by_definition(e_rows):
    rows, nb = e_rows.shape
    out = np.full(rows * nb, 255, np.uint8)
    pos = 0
    for p in range(0, nb, 8):
        w = min(8, nb - p)
        order = list(range(0, w, 2)) + list(range(1, w, 2))    # even blocks first
        for r in range(rows):
            for j in order:
                out[pos] = e_rows[r, p + j]
                pos += 1
    assert pos == rows * nb
    return out


@pytest.mark.parametrize("rows,K", [(1, 32), (3, 384), (5, 256), (2, 96), (7, 1152), (4, 2048)])
def test_mxfp4_panel_layout(rows, K):
    rng = np.random.default_rng(rows * 1000 + K)
    e_rows = rng.integers(0, 255, size=(rows, K // 32), dtype=np.uint8)
    want = panels_by_definition(e_rows)
    assert np.array_equal(ops.mxfp4_scales_to_panels(e_rows), want)
    assert np.array_equal(ops.mxfp4_scales_to_rows(want, rows, K), e_rows)
    offs = ops.mxfp4_scale_offsets(rows, K).numpy()
    assert sorted(offs.reshape(-1).tolist()) == list(range(rows * (K // 32)))   # a permutation


def test_mxfp4_panel_layout_torch():
    import torch
    e_rows = torch.arange(6 * 12, dtype=torch.int64).reshape(6, 12).to(torch.uint8)
    flat = ops.mxfp4_scales_to_panels(e_rows)
    assert torch.equal(ops.mxfp4_scales_to_rows(flat, 6, 384), e_rows)
    assert np.array_equal(flat.numpy(), panels_by_definition(e_rows.numpy()))


def nv_panels_by_definition(s_rows):
    """The NVFP4 scale panel layout written out with loops from its definition:
    panel p = blocks 16p..16p+15, rows of 16 bytes, the blocks in the order
    0,1,4,5,8,9,12,13,2,3,6,7,10,11,14,15."""
    rows, nb = s_rows.shape
    order = [0, 1, 4, 5, 8, 9, 12, 13, 2, 3, 6, 7, 10, 11, 14, 15]
    out = []
    for p in range(nb // 16):
        for r in range(rows):
            for j in order:
                out.append(s_rows[r, 16 * p + j])
    return np.array(out, dtype=s_rows.dtype)


@pytest.mark.parametrize("rows,K", [(1, 256), (5, 512), (3, 3584)])
def test_nvfp4_panel_layout(rows, K):
    rng = np.random.default_rng(rows + K)
    s_rows = rng.integers(0, 256, (rows, K // 16), dtype=np.uint8)
    flat = ops.nvfp4_scales_to_panels(s_rows)
    assert np.array_equal(flat, nv_panels_by_definition(s_rows))
    assert np.array_equal(ops.nvfp4_scales_to_rows(flat, rows, K), s_rows)
