"""Tensor-level wrappers over the C ABI (same names as include/w4a4.h).

Each wrapper checks dtypes/devices, allocates outputs with torch on the input's
device and calls the library on torch's current stream. Nothing is computed
here.
"""
from __future__ import annotations

import torch

from ._lib import Y_F16, Y_F32, call


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t: torch.Tensor, dtype, name: str) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _ydtype(dtype) -> int:
    if dtype == torch.float32:
        return Y_F32
    if dtype == torch.float16:
        return Y_F16
    raise TypeError("output dtype must be torch.float32 or torch.float16")


def _need_scales(s: torch.Tensor, K: int, group: int, rows: int, name: str) -> None:
    """Group-major INT4 scales: contiguous, K/group x rows floats."""
    if group > 0 and K % group == 0 and (not s.is_contiguous() or s.numel() != (K // group) * rows):
        raise ValueError(f"{name} must be contiguous group-major scales [K/group, rows]")


def w4a4_quantize_act(x: torch.Tensor, group: int = 128, out=None):
    """INT4 group quantization of fp16 X[M, K] (row stride may exceed K).

    Returns ``(xq uint8 [M, K/2], xs float32 [K/group, M])``: the scales are
    group-major (``xs[c, m]`` is the scale of row m, group c).
    """
    _need(x, torch.float16, "x")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    M, K = x.shape
    if out is None:
        xq = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
        xs = torch.empty((max(K // max(group, 1), 0), M), dtype=torch.float32, device=x.device)
    else:
        xq, xs = out
    call("w4a4_quantize_act", x.data_ptr(), M, K, x.stride(0), group,
         xq.data_ptr(), xs.data_ptr(), _stream(x))
    return xq, xs


def w4a4_pack_weight(w: torch.Tensor, group: int = 128, out=None):
    """Offline INT4 group quantization of fp16 W[N, K] (contiguous):
    ``(wq uint8 [N, K/2], ws float32 [K/group, N])``, scales group-major."""
    _need(w, torch.float16, "w")
    if w.dim() != 2 or not w.is_contiguous():
        raise ValueError("w must be a contiguous 2-D tensor")
    N, K = w.shape
    if out is None:
        wq = torch.empty((N, K // 2), dtype=torch.uint8, device=w.device)
        ws = torch.empty((max(K // max(group, 1), 0), N), dtype=torch.float32, device=w.device)
    else:
        wq, ws = out
    call("w4a4_pack_weight", w.data_ptr(), N, K, group, wq.data_ptr(), ws.data_ptr(), _stream(w))
    return wq, ws


def w4a4_gemm(xq, xs, group_a: int, wq, ws, group_w: int, out_dtype=torch.float32, out=None):
    """Y[M, N] = group-dequantized INT4 GEMM of packed X and W."""
    for t, dt, n in ((xq, torch.uint8, "xq"), (wq, torch.uint8, "wq"),
                     (xs, torch.float32, "xs"), (ws, torch.float32, "ws")):
        _need(t, dt, n)
    M, K = xq.shape[0], xq.shape[1] * 2
    N = wq.shape[0]
    if wq.shape[1] * 2 != K:
        raise ValueError("K of xq and wq differ")
    _need_scales(xs, K, group_a, M, "xs")
    _need_scales(ws, K, group_w, N, "ws")
    y = torch.empty((M, N), dtype=out_dtype, device=xq.device) if out is None else out
    call("w4a4_gemm", xq.data_ptr(), xs.data_ptr(), group_a, wq.data_ptr(), ws.data_ptr(), group_w,
         M, N, K, y.data_ptr(), _ydtype(y.dtype), y.stride(0), _stream(xq))
    return y


def w4a4_gemm_splitk(xq, xs, group_a: int, wq, ws, group_w: int, splits: int = 0,
                     out_dtype=torch.float32, out=None, workspace=None):
    """w4a4_gemm with K split across workgroups (``splits=0``: the library
    picks). The fp32 workspace is allocated here with torch unless given."""
    from ._lib import splitk_workspace_bytes
    for t, n in ((xq, "xq"), (wq, "wq")):
        _need(t, torch.uint8, n)
    _need(xs, torch.float32, "xs")
    _need(ws, torch.float32, "ws")
    M, K = xq.shape[0], xq.shape[1] * 2
    N = wq.shape[0]
    if wq.shape[1] * 2 != K:
        raise ValueError("K of xq and wq differ")
    _need_scales(xs, K, group_a, M, "xs")
    _need_scales(ws, K, group_w, N, "ws")
    nbytes = splitk_workspace_bytes(M, N, K, group_a, group_w, splits)
    if workspace is None:
        workspace = torch.empty((max(nbytes, 16) // 4,), dtype=torch.float32, device=xq.device)
    elif workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace must hold {nbytes} bytes")
    y = torch.empty((M, N), dtype=out_dtype, device=xq.device) if out is None else out
    call("w4a4_gemm_splitk", xq.data_ptr(), xs.data_ptr(), group_a, wq.data_ptr(), ws.data_ptr(), group_w,
         M, N, K, splits, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
         y.data_ptr(), _ydtype(y.dtype), y.stride(0), _stream(xq))
    return y


def w4a4_gemm_debug_partials(xq, xs, group_a: int, wq, ws, group_w: int, m0: int, mc: int, n0: int, nc: int):
    """Exact int32 group partials P_b for the window; shape [K/g, mc, nc]."""
    M, K = xq.shape[0], xq.shape[1] * 2
    N = wq.shape[0]
    g = min(group_a, group_w)
    part = torch.empty((K // g, mc, nc), dtype=torch.int32, device=xq.device)
    call("w4a4_gemm_debug_partials", xq.data_ptr(), xs.data_ptr(), group_a, wq.data_ptr(), ws.data_ptr(),
         group_w, M, N, K, m0, mc, n0, nc, part.data_ptr(), _stream(xq))
    return part


def mxfp4_scale_offsets(rows: int, K: int):
    """Byte offset of the scale of (row r, block b) in the 256-k panel layout
    of the C header: ``8*rows*p + w_p*r + pos`` with ``p = b // 8``,
    ``w_p = min(8, K/32 - 8p)``, ``j = b % 8`` and ``pos = j // 2`` for even
    j, ``ceil(w_p / 2) + j // 2`` for odd j. Returns an int64 tensor [rows, K/32]."""
    nb = K // 32
    b = torch.arange(nb, dtype=torch.int64)
    p = b // 8
    w = torch.clamp(nb - 8 * p, max=8)
    j = b % 8
    pos = torch.where(j % 2 == 0, j // 2, (w + 1) // 2 + j // 2)
    r = torch.arange(rows, dtype=torch.int64)[:, None]
    return 8 * rows * p[None, :] + w[None, :] * r + pos[None, :]


def mxfp4_scales_to_rows(e, rows: int, K: int):
    """Panel-layout scale bytes (flat, ``rows*K/32``) -> row-major [rows, K/32]
    (torch tensor on its device, or numpy array)."""
    idx = mxfp4_scale_offsets(rows, K)
    if isinstance(e, torch.Tensor):
        return e.reshape(-1)[idx.to(e.device)]
    return e.reshape(-1)[idx.numpy()]


def mxfp4_scales_to_panels(e_rows):
    """Row-major [rows, K/32] scale bytes -> the flat panel layout."""
    rows, nb = e_rows.shape
    idx = mxfp4_scale_offsets(rows, 32 * nb).reshape(-1)
    if isinstance(e_rows, torch.Tensor):
        out = torch.empty(rows * nb, dtype=e_rows.dtype, device=e_rows.device)
        out[idx.to(e_rows.device)] = e_rows.reshape(-1)
        return out
    import numpy as np
    out = np.empty(rows * nb, dtype=e_rows.dtype)
    out[idx.numpy()] = e_rows.reshape(-1)
    return out


def mxfp4_quantize(x: torch.Tensor, out=None):
    """MXFP4 quantization of fp16 X[rows, K]: ``(codes uint8 [rows, K/2],
    e8m0 uint8 [rows*K/32] in the 256-k panel layout)``; see
    :func:`mxfp4_scales_to_rows` for the row-major view."""
    _need(x, torch.float16, "x")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    R, K = x.shape
    if out is None:
        q = torch.empty((R, K // 2), dtype=torch.uint8, device=x.device)
        e = torch.empty((R * (K // 32),), dtype=torch.uint8, device=x.device)
    else:
        q, e = out
    if e.numel() != R * (K // 32) or not e.is_contiguous():
        raise ValueError("e8m0 must be contiguous with rows*K/32 bytes")
    call("mxfp4_quantize", x.data_ptr(), R, K, x.stride(0), q.data_ptr(), e.data_ptr(), _stream(x))
    return q, e


def _mxfp4_quantize_wide(fn: str, x: torch.Tensor, out):
    _need(x, torch.float16, "x")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    R, K = x.shape
    if out is None:
        q = torch.empty((R, K), dtype=torch.uint8, device=x.device)
        e = torch.empty((R * (2 * K // 32),), dtype=torch.uint8, device=x.device)
    else:
        q, e = out
    if e.numel() != R * (2 * K // 32) or not e.is_contiguous():
        raise ValueError("e8m0 must be contiguous with rows*2K/32 bytes")
    call(fn, x.data_ptr(), R, K, x.stride(0), q.data_ptr(), e.data_ptr(), _stream(x))
    return q, e


def mxfp4_quantize_residual(x: torch.Tensor, out=None):
    """Two-pass MXFP4 with the residual appended along K: ``(codes uint8
    [rows, K] (2K codes: Q(x) then Q(x - deq Q(x))), e8m0 uint8 [rows*2K/32]
    in the panel layout of a 2K-wide matrix)``."""
    return _mxfp4_quantize_wide("mxfp4_quantize_residual", x, out)


def mxfp4_quantize_append_copy(w: torch.Tensor, out=None):
    """``[Q(w) | Q(w)]`` along K (shapes as :func:`mxfp4_quantize_residual`):
    the weight side of the appended-residual GEMM."""
    return _mxfp4_quantize_wide("mxfp4_quantize_append_copy", w, out)


def mxfp4_gemm(xq, xe, wq, we, out_dtype=torch.float32, out=None):
    """Y[M, N] = block-scaled FP4 GEMM of MXFP4 X and W."""
    for t, n in ((xq, "xq"), (xe, "xe"), (wq, "wq"), (we, "we")):
        _need(t, torch.uint8, n)
    M, K = xq.shape[0], xq.shape[1] * 2
    N = wq.shape[0]
    if wq.shape[1] * 2 != K:
        raise ValueError("K of xq and wq differ")
    if xe.numel() != M * (K // 32) or we.numel() != N * (K // 32):
        raise ValueError("scale tensors must hold rows*K/32 bytes (panel layout)")
    y = torch.empty((M, N), dtype=out_dtype, device=xq.device) if out is None else out
    call("mxfp4_gemm", xq.data_ptr(), xe.data_ptr(), wq.data_ptr(), we.data_ptr(), M, N, K,
         y.data_ptr(), _ydtype(y.dtype), y.stride(0), _stream(xq))
    return y


def mxfp4_gemm_debug_partials(xq, xe, wq, we, m0: int, mc: int, n0: int, nc: int):
    """Exact int32 block integers I_b = sum (2va)(2vw) for the window; [K/32, mc, nc]."""
    M, K = xq.shape[0], xq.shape[1] * 2
    N = wq.shape[0]
    part = torch.empty((K // 32, mc, nc), dtype=torch.int32, device=xq.device)
    call("mxfp4_gemm_debug_partials", xq.data_ptr(), xe.data_ptr(), wq.data_ptr(), we.data_ptr(),
         M, N, K, m0, mc, n0, nc, part.data_ptr(), _stream(xq))
    return part


# ------------------------------------------------------------------- NVFP4

def nvfp4_scale_offsets(rows: int, K: int):
    """Byte offset of the E4M3 scale of (row r, block b) in the 256-k panel
    layout of the C header: ``16*rows*p + 16*r + 8*((j>>1)&1) + 2*(j>>2) +
    (j&1)`` with ``p = b // 16``, ``j = b % 16``. Returns int64 [rows, K/16]."""
    b = torch.arange(K // 16, dtype=torch.int64)
    p, j = b // 16, b % 16
    pos = 8 * ((j >> 1) & 1) + 2 * (j >> 2) + (j & 1)
    r = torch.arange(rows, dtype=torch.int64)[:, None]
    return 16 * rows * p[None, :] + 16 * r + pos[None, :]


def nvfp4_scales_to_rows(s, rows: int, K: int):
    """Panel-layout scale bytes (flat, ``rows*K/16``) -> row-major [rows, K/16]
    (torch tensor on its device, or numpy array)."""
    idx = nvfp4_scale_offsets(rows, K)
    if isinstance(s, torch.Tensor):
        return s.reshape(-1)[idx.to(s.device)]
    return s.reshape(-1)[idx.numpy()]


def nvfp4_scales_to_panels(s_rows):
    """Row-major [rows, K/16] scale bytes -> the flat panel layout."""
    rows, nb = s_rows.shape
    idx = nvfp4_scale_offsets(rows, 16 * nb).reshape(-1)
    if isinstance(s_rows, torch.Tensor):
        out = torch.empty(rows * nb, dtype=s_rows.dtype, device=s_rows.device)
        out[idx.to(s_rows.device)] = s_rows.reshape(-1)
        return out
    import numpy as np
    out = np.empty(rows * nb, dtype=s_rows.dtype)
    out[idx.numpy()] = s_rows.reshape(-1)
    return out


def _need_scalar(t, name: str) -> None:
    _need(t, torch.float32, name)
    if t.numel() != 1:
        raise ValueError(f"{name} must hold one float")


def nvfp4_global_scale(x: torch.Tensor, out=None):
    """``fl32(max|x| / 2688)`` of fp16 X[rows, K] as a one-element float32
    tensor on the device (computed there, no host sync)."""
    _need(x, torch.float16, "x")
    if x.dim() != 2 or (x.shape[0] > 0 and x.stride(1) != 1):
        raise ValueError("x must be 2-D with unit column stride")
    g = torch.empty((1,), dtype=torch.float32, device=x.device) if out is None else out
    _need_scalar(g, "out")
    ldx = x.stride(0) if x.shape[0] > 0 else x.shape[1]
    call("nvfp4_global_scale", x.data_ptr(), x.shape[0], x.shape[1], ldx, g.data_ptr(), _stream(x))
    return g


def nvfp4_quantize(x: torch.Tensor, global_scale: torch.Tensor, out=None):
    """NVFP4 quantization of fp16 X[rows, K] with a device global scale:
    ``(codes uint8 [rows, K/2], E4M3 scales uint8 [rows*K/16] in the 256-k
    panel layout)``; see :func:`nvfp4_scales_to_rows`."""
    _need(x, torch.float16, "x")
    _need_scalar(global_scale, "global_scale")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    R, K = x.shape
    if out is None:
        q = torch.empty((R, K // 2), dtype=torch.uint8, device=x.device)
        s = torch.empty((R * (K // 16),), dtype=torch.uint8, device=x.device)
    else:
        q, s = out
    if s.numel() != R * (K // 16) or not s.is_contiguous():
        raise ValueError("scales must be contiguous with rows*K/16 bytes")
    call("nvfp4_quantize", x.data_ptr(), R, K, x.stride(0), global_scale.data_ptr(),
         q.data_ptr(), s.data_ptr(), _stream(x))
    return q, s


def _nv_shapes(xq, xs, wq, ws):
    for t, n in ((xq, "xq"), (xs, "xs"), (wq, "wq"), (ws, "ws")):
        _need(t, torch.uint8, n)
    M, K = xq.shape[0], xq.shape[1] * 2
    N = wq.shape[0]
    if wq.shape[1] * 2 != K:
        raise ValueError("K of xq and wq differ")
    if xs.numel() != M * (K // 16) or ws.numel() != N * (K // 16):
        raise ValueError("scale tensors must hold rows*K/16 bytes (panel layout)")
    return M, N, K


def nvfp4_gemm(xq, xs, x_global, wq, ws, w_global, out_dtype=torch.float32, out=None):
    """Y[M, N] = NVFP4 GEMM of X and W (fp16 matrix cores, fp32 accumulation)."""
    M, N, K = _nv_shapes(xq, xs, wq, ws)
    _need_scalar(x_global, "x_global")
    _need_scalar(w_global, "w_global")
    y = torch.empty((M, N), dtype=out_dtype, device=xq.device) if out is None else out
    call("nvfp4_gemm", xq.data_ptr(), xs.data_ptr(), x_global.data_ptr(), wq.data_ptr(), ws.data_ptr(),
         w_global.data_ptr(), M, N, K, y.data_ptr(), _ydtype(y.dtype), y.stride(0), _stream(xq))
    return y


def nvfp4_gemm_debug_partials(xq, xs, wq, ws, m0: int, mc: int, n0: int, nc: int):
    """Exact int32 block integers I_b = sum (2vx)(2vw) over 16-blocks; [K/16, mc, nc]."""
    M, N, K = _nv_shapes(xq, xs, wq, ws)
    part = torch.empty((K // 16, mc, nc), dtype=torch.int32, device=xq.device)
    call("nvfp4_gemm_debug_partials", xq.data_ptr(), xs.data_ptr(), wq.data_ptr(), ws.data_ptr(),
         M, N, K, m0, mc, n0, nc, part.data_ptr(), _stream(xq))
    return part
