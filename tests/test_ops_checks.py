"""Host-side checks of caller-supplied buffers in the tensor wrappers (CPU only).

The C ABI sees raw pointers, not buffer sizes, so the wrappers must refuse an
output buffer of the wrong shape, dtype, device or stride before the call:
otherwise a kernel would write past the allocation. These tests run the
checks on CPU tensors (the device every tensor here has); the GPU parity
tests exercise the same wrappers end to end.
"""
import pytest
import torch

from w4a4_quantized_gemm_quantize_amd import ops

CPU = torch.device("cpu")


def test_check_out_accepts_exact_buffer():
    ops._check_out(torch.empty(4, 8, dtype=torch.uint8), "q", (4, 8), torch.uint8, CPU)
    ops._check_out(torch.empty(3, 5, dtype=torch.float32), "s", (3, 5), torch.float32, CPU)


@pytest.mark.parametrize("bad, exc", [
    (torch.empty(4, 7, dtype=torch.uint8), ValueError),          # too small
    (torch.empty(5, 8, dtype=torch.uint8), ValueError),          # too many rows
    (torch.empty(32, dtype=torch.uint8), ValueError),            # right size, wrong shape
    (torch.empty(4, 8, dtype=torch.int8), TypeError),            # wrong dtype
    (torch.empty(8, 4, dtype=torch.uint8).t(), ValueError),      # not contiguous
    (torch.empty(4, 16, dtype=torch.uint8)[:, :8], ValueError),  # strided view
    (None, TypeError),
])
def test_check_out_rejects(bad, exc):
    with pytest.raises(exc):
        ops._check_out(bad, "q", (4, 8), torch.uint8, CPU)


def test_check_out_rejects_foreign_device():
    with pytest.raises(ValueError):
        ops._check_out(torch.empty(4, 8, dtype=torch.uint8), "q", (4, 8), torch.uint8, torch.device("meta"))


def test_y_out_rules():
    y = ops._y_out(None, 3, 5, torch.float16, CPU)
    assert y.shape == (3, 5) and y.dtype == torch.float16
    big = torch.empty(3, 9, dtype=torch.float32)
    assert ops._y_out(big[:, :5], 3, 5, None, CPU).stride(0) == 9   # row stride >= N is allowed
    with pytest.raises(ValueError):
        ops._y_out(torch.empty(3, 4, dtype=torch.float32), 3, 5, None, CPU)
    with pytest.raises(ValueError):
        ops._y_out(torch.empty(2, 5, dtype=torch.float32), 3, 5, None, CPU)
    with pytest.raises(ValueError):
        ops._y_out(torch.empty(5, 3, dtype=torch.float32).t(), 3, 5, None, CPU)   # column stride 3
    with pytest.raises(TypeError):
        ops._y_out(torch.empty(3, 5, dtype=torch.float64), 3, 5, None, CPU)
    with pytest.raises(ValueError):
        ops._y_out(torch.empty(3, 5, dtype=torch.float32), 3, 5, None, torch.device("meta"))


def test_wrappers_refuse_host_tensors():
    x = torch.zeros(4, 256, dtype=torch.float16)
    with pytest.raises(TypeError):
        ops.w4a4_quantize_act(x, 128)
    with pytest.raises(TypeError):
        ops.mxfp4_quantize(x)
    q = torch.zeros(4, 128, dtype=torch.uint8)
    s = torch.zeros(2, 4, dtype=torch.float32)
    with pytest.raises(TypeError):
        ops.w4a4_gemm_debug_partials(q, s, 128, q, s, 128, 0, 1, 0, 1)
