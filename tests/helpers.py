"""Shared helpers for the GPU parity tests (no arithmetic of the method here)."""
import numpy as np

RTOL = 1e-5   # |Y_gpu - Y| <= RTOL * T + ATOL, T = sum of |group terms|
ATOL = 1e-6


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_y_close(y_gpu, Y, T, what=""):
    """fp32 output within the per-element tolerance; returns max |err|/bound."""
    y = np.asarray(y_gpu, dtype=np.float64)
    bound = RTOL * T + ATOL
    err = np.abs(y - Y)
    ratio = float((err / bound).max()) if err.size else 0.0
    bad = np.argwhere(err > bound)
    assert bad.size == 0, (f"{what}: {len(bad)} elements out of tolerance, first {bad[:5].tolist()}, "
                           f"max ratio {ratio:.3g}")
    return ratio


def assert_y16_close(y16, Y, T, what=""):
    """fp16 output: within one fp16 ulp of fp16(Y) plus the fp32 tolerance."""
    y = np.asarray(y16, dtype=np.float64)
    ref16 = Y.astype(np.float16)
    a = np.abs(ref16.astype(np.float64))
    ulp = np.spacing(np.maximum(a, np.float64(np.finfo(np.float16).tiny)).astype(np.float16)).astype(np.float64)
    bound = ulp + RTOL * T + ATOL
    err = np.abs(y - Y)
    bad = np.argwhere(err > bound)
    assert bad.size == 0, f"{what}: {len(bad)} fp16 elements out of tolerance, first {bad[:5].tolist()}"
