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


def _check_out(t, name: str, shape, dtype, device, row_stride_ok: bool = False) -> None:
    """A caller-supplied output buffer must have exactly the shape, dtype and
    device the kernel writes (the C ABI cannot see buffer sizes: an undersized
    or foreign buffer would be written past its end). ``row_stride_ok``: a 2-D
    output may have a row stride above its width (unit column stride)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if row_stride_ok and t.dim() == 2:
        if t.numel() and (t.stride(1) != 1 or t.stride(0) < t.shape[1]):
            raise ValueError(f"{name} must have unit column stride and row stride >= its width")
    elif not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _y_out(out, M: int, N: int, out_dtype, device) -> torch.Tensor:
    """The GEMM output: a new [M, N] tensor, or the caller's, checked (fp32 or
    fp16, [M, N] on the inputs' device, unit column stride, row stride >= N)."""
    if out is None:
        return torch.empty((M, N), dtype=out_dtype, device=device)
    _ydtype(out.dtype)
    _check_out(out, "out", (M, N), out.dtype, device, row_stride_ok=True)
    return out


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
        _check_out(xq, "xq", (M, K // 2), torch.uint8, x.device)
        _check_out(xs, "xs", (K // max(group, 1), M), torch.float32, x.device)
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
        _check_out(wq, "wq", (N, K // 2), torch.uint8, w.device)
        _check_out(ws, "ws", (K // max(group, 1), N), torch.float32, w.device)
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
    y = _y_out(out, M, N, out_dtype, xq.device)
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
    else:
        if not isinstance(workspace, torch.Tensor) or workspace.device != xq.device:
            raise ValueError("workspace must be a tensor on the inputs' device")
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace must hold {nbytes} bytes")
    y = _y_out(out, M, N, out_dtype, xq.device)
    call("w4a4_gemm_splitk", xq.data_ptr(), xs.data_ptr(), group_a, wq.data_ptr(), ws.data_ptr(), group_w,
         M, N, K, splits, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
         y.data_ptr(), _ydtype(y.dtype), y.stride(0), _stream(xq))
    return y


# When w4a4_linear picks the fused launch by itself. The fused launch saves the
# activation quantizer's launch (about 5 us per linear at decode), but each of
# its workgroups re-reads and re-quantizes all of X: on 16-column tiles that
# is M/4 of the weight bytes again through L2, so its cost grows as M times the
# GEMM's own time. Measured FFN decode steps, fused against quantize + GEMM:
# LLaMA-2-70B (112 MiB of weights per linear) faster fused up to M = 3, slower
# at M = 4; LLaMA-2-7B (21.5 MiB) faster up to M = 4, even at M = 6, slower at
# M = 8. The rule M x (weight bytes + FUSED_FIXED_BYTES) <= FUSED_BUDGET_BYTES
# (the fixed term stands for the GEMM's latency, which does not shrink with
# the weights) takes M <= 3 and M <= 5 there; the kernel's own LDS limit
# (w4a4_linear_fused_supported) applies on top.
FUSED_FIXED_BYTES = 96 << 20
FUSED_BUDGET_BYTES = 640 << 20


def use_fused(M: int, N: int, K: int, group_a: int, group_w: int) -> bool:
    """Whether w4a4_linear takes the fused launch for this shape by default."""
    from ._lib import load_library
    return (M > 0 and N > 0 and M * (N * K // 2 + FUSED_FIXED_BYTES) <= FUSED_BUDGET_BYTES and
            bool(load_library().w4a4_linear_fused_supported(M, N, K, group_a, group_w)))


def w4a4_linear(x: torch.Tensor, wq, ws, group_a: int = 128, group_w: int = 128, out_dtype=torch.float32,
                out=None, fused: bool | None = None):
    """A W4A4 linear layer on fp16 activations: Y = Q(X) Q(W)^T with X quantized
    per group of ``group_a`` here. For few tokens (tiny M x K) one fused launch
    quantizes and multiplies (``w4a4_linear_fused``); otherwise the activation
    quantizer runs first and the GEMM (with its automatic K split) after it.
    ``fused``: None picks (:func:`use_fused`), True requires the fused path,
    False forbids it."""
    from ._lib import load_library
    _need(x, torch.float16, "x")
    _need(wq, torch.uint8, "wq")
    _need(ws, torch.float32, "ws")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    M, K = x.shape
    N = wq.shape[0]
    if wq.shape[1] * 2 != K:
        raise ValueError("K of x and wq differ")
    _need_scales(ws, K, group_w, N, "ws")
    ok = M > 0 and N > 0 and bool(load_library().w4a4_linear_fused_supported(M, N, K, group_a, group_w))
    if fused and not ok:
        raise ValueError(f"the fused path does not take M={M} N={N} K={K} group_a={group_a}")
    if fused is None:
        fused = use_fused(M, N, K, group_a, group_w)
    if fused:
        y = _y_out(out, M, N, out_dtype, x.device)
        call("w4a4_linear_fused", x.data_ptr(), M, K, x.stride(0), group_a, wq.data_ptr(), ws.data_ptr(),
             group_w, N, y.data_ptr(), _ydtype(y.dtype), y.stride(0), _stream(x))
        return y
    xq, xs = w4a4_quantize_act(x, group_a)
    return w4a4_gemm_splitk(xq, xs, group_a, wq, ws, group_w, out_dtype=out_dtype, out=out)


def w4a4_gemm_debug_partials(xq, xs, group_a: int, wq, ws, group_w: int, m0: int, mc: int, n0: int, nc: int):
    """Exact int32 group partials P_b for the window; shape [K/g, mc, nc]."""
    for t, dt, n in ((xq, torch.uint8, "xq"), (wq, torch.uint8, "wq"),
                     (xs, torch.float32, "xs"), (ws, torch.float32, "ws")):
        _need(t, dt, n)
    M, K = xq.shape[0], xq.shape[1] * 2
    N = wq.shape[0]
    if wq.shape[1] * 2 != K:
        raise ValueError("K of xq and wq differ")
    _need_scales(xs, K, group_a, M, "xs")
    _need_scales(ws, K, group_w, N, "ws")
    g = min(group_a, group_w)
    if g <= 0 or K % g:
        raise ValueError("the finer group must divide K")
    part = torch.empty((K // g, mc, nc), dtype=torch.int32, device=xq.device)
    call("w4a4_gemm_debug_partials", xq.data_ptr(), xs.data_ptr(), group_a, wq.data_ptr(), ws.data_ptr(),
         group_w, M, N, K, m0, mc, n0, nc, part.data_ptr(), _stream(xq))
    return part


def mxfp4_quantize(x: torch.Tensor, out=None):
    """MXFP4 quantization of fp16 X[rows, K]: ``(codes uint8 [rows, K/2],
    e8m0 uint8 [rows*K/32] in the 256-k panel layout)``; see
    :func:`mxfp4_scales_to_rows` for the row-major form."""
    _need(x, torch.float16, "x")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    R, K = x.shape
    if out is None:
        q = torch.empty((R, K // 2), dtype=torch.uint8, device=x.device)
        e = torch.empty((R * (K // 32),), dtype=torch.uint8, device=x.device)
    else:
        q, e = out
        _check_out(q, "codes", (R, K // 2), torch.uint8, x.device)
        _check_out(e, "e8m0", (R * (K // 32),), torch.uint8, x.device)
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
        _check_out(q, "codes", (R, K), torch.uint8, x.device)
        _check_out(e, "e8m0", (R * (2 * K // 32),), torch.uint8, x.device)
    call(fn, x.data_ptr(), R, K, x.stride(0), q.data_ptr(), e.data_ptr(), _stream(x))
    return q, e


def mxfp4_quantize_residual(x: torch.Tensor, out=None):
    """Two-pass MXFP4 with the residual appended along K: ``(codes uint8
    [rows, K] (2K codes: Q(x) then Q(x - deq Q(x))), e8m0 uint8 [rows*2K/32]
    in the panel layout of a 2K-wide matrix)``."""
    return _mxfp4_quantize_wide("mxfp4_quantize_residual", x, out)


def mxfp4_quantize_residual_tied(x: torch.Tensor, out=None):
    """Two-pass MXFP4 with the second scale tied to the first (no clipping in
    either pass; per-element error <= 2^(E1 + 3) / 64): shapes and layouts as
    :func:`mxfp4_quantize_residual`."""
    return _mxfp4_quantize_wide("mxfp4_quantize_residual_tied", x, out)


def mxfp4_quantize_append_copy(w: torch.Tensor, out=None):
    """``[Q(w) | Q(w)]`` along K (shapes as :func:`mxfp4_quantize_residual`):
    the weight side of the appended-residual GEMM."""
    return _mxfp4_quantize_wide("mxfp4_quantize_append_copy", w, out)


def _mx_shapes(xq, xe, wq, we):
    for t, n in ((xq, "xq"), (xe, "xe"), (wq, "wq"), (we, "we")):
        _need(t, torch.uint8, n)
    M, K = xq.shape[0], xq.shape[1] * 2
    N = wq.shape[0]
    if wq.shape[1] * 2 != K:
        raise ValueError("K of xq and wq differ")
    if xe.numel() != M * (K // 32) or we.numel() != N * (K // 32):
        raise ValueError("scale tensors must hold rows*K/32 bytes (panel layout)")
    return M, N, K


def mxfp4_gemm(xq, xe, wq, we, out_dtype=torch.float32, out=None):
    """Y[M, N] = block-scaled FP4 GEMM of MXFP4 X and W."""
    M, N, K = _mx_shapes(xq, xe, wq, we)
    y = _y_out(out, M, N, out_dtype, xq.device)
    call("mxfp4_gemm", xq.data_ptr(), xe.data_ptr(), wq.data_ptr(), we.data_ptr(), M, N, K,
         y.data_ptr(), _ydtype(y.dtype), y.stride(0), _stream(xq))
    return y


def mxfp4_gemm_debug_partials(xq, xe, wq, we, m0: int, mc: int, n0: int, nc: int):
    """Exact int32 block integers I_b = sum (2va)(2vw) for the window; [K/32, mc, nc]."""
    M, N, K = _mx_shapes(xq, xe, wq, we)
    part = torch.empty((K // 32, mc, nc), dtype=torch.int32, device=xq.device)
    call("mxfp4_gemm_debug_partials", xq.data_ptr(), xe.data_ptr(), wq.data_ptr(), we.data_ptr(),
         M, N, K, m0, mc, n0, nc, part.data_ptr(), _stream(xq))
    return part


# ------------------------------------------------------------------- NVFP4

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
    _check_out(g, "out", (1,), torch.float32, x.device)
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
        _check_out(q, "codes", (R, K // 2), torch.uint8, x.device)
        _check_out(s, "scales", (R * (K // 16),), torch.uint8, x.device)
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
    y = _y_out(out, M, N, out_dtype, xq.device)
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


# -------------------------------------------------------- storage conversions
# Canonical storage (two's-complement INT4 nibbles, row-major scales) <-> the
# layouts the GEMMs read; every conversion runs in the library's kernels.

def w4a4_repack_int4(nibbles: torch.Tensor, check: bool = True):
    """Canonical INT4 codes (uint8 [rows, K/2], two's-complement nibbles, even
    k low) -> the GEMM's INT4 layout. Returns ``(packed, minus8_count)``, the
    count a one-element int32 device tensor. With ``check`` (default) the call
    synchronizes and raises if any code is -8 (no sign-magnitude form)."""
    _need(nibbles, torch.uint8, "nibbles")
    if nibbles.dim() != 2 or not nibbles.is_contiguous():
        raise ValueError("nibbles must be a contiguous 2-D tensor")
    rows, K = nibbles.shape[0], nibbles.shape[1] * 2
    packed = torch.empty_like(nibbles)
    count = torch.empty((1,), dtype=torch.int32, device=nibbles.device)
    call("w4a4_repack_int4", nibbles.data_ptr(), rows, K, packed.data_ptr(), count.data_ptr(), _stream(nibbles))
    if check and int(count.item()) != 0:
        raise ValueError(f"{int(count.item())} INT4 codes are -8: the GEMM layout holds [-7, 7] only")
    return packed, count


def w4a4_unpack_int4(packed: torch.Tensor):
    """The GEMM's INT4 layout -> canonical two's-complement nibbles (-0 -> 0)."""
    _need(packed, torch.uint8, "packed")
    if packed.dim() != 2 or not packed.is_contiguous():
        raise ValueError("packed must be a contiguous 2-D tensor")
    out = torch.empty_like(packed)
    call("w4a4_unpack_int4", packed.data_ptr(), packed.shape[0], packed.shape[1] * 2, out.data_ptr(),
         _stream(packed))
    return out


def w4a4_scales_to_group_major(scales_rows: torch.Tensor):
    """Row-major INT4 scales float32 [rows, groups] -> group-major [groups, rows]."""
    _need(scales_rows, torch.float32, "scales_rows")
    if scales_rows.dim() != 2 or not scales_rows.is_contiguous():
        raise ValueError("scales_rows must be a contiguous 2-D tensor")
    rows, groups = scales_rows.shape
    out = torch.empty((groups, rows), dtype=torch.float32, device=scales_rows.device)
    call("w4a4_scales_to_group_major", scales_rows.data_ptr(), rows, groups, out.data_ptr(), _stream(scales_rows))
    return out


def w4a4_scales_to_row_major(scales_gm: torch.Tensor):
    """Group-major INT4 scales float32 [groups, rows] -> row-major [rows, groups]."""
    _need(scales_gm, torch.float32, "scales_gm")
    if scales_gm.dim() != 2 or not scales_gm.is_contiguous():
        raise ValueError("scales_gm must be a contiguous 2-D tensor")
    groups, rows = scales_gm.shape
    out = torch.empty((rows, groups), dtype=torch.float32, device=scales_gm.device)
    call("w4a4_scales_to_row_major", scales_gm.data_ptr(), rows, groups, out.data_ptr(), _stream(scales_gm))
    return out


def _panels(fn: str, src: torch.Tensor, rows: int, K: int, block: int, to_panels: bool):
    _need(src, torch.uint8, "scales")
    if not src.is_contiguous() or src.numel() != rows * (K // block):
        raise ValueError(f"scales must be contiguous with rows*K/{block} bytes")
    shape = (rows * (K // block),) if to_panels else (rows, K // block)
    out = torch.empty(shape, dtype=torch.uint8, device=src.device)
    call(fn, src.data_ptr(), rows, K, out.data_ptr(), _stream(src))
    return out


def mxfp4_scales_to_panels(e_rows: torch.Tensor):
    """Row-major E8M0 bytes [rows, K/32] -> the flat 256-k panel layout."""
    rows, nb = e_rows.shape
    return _panels("mxfp4_scales_to_panels", e_rows, rows, 32 * nb, 32, True)


def mxfp4_scales_to_rows(e: torch.Tensor, rows: int, K: int):
    """Panel-layout E8M0 bytes (flat, rows*K/32) -> row-major [rows, K/32]."""
    return _panels("mxfp4_scales_to_rows", e, rows, K, 32, False)


def nvfp4_scales_to_panels(s_rows: torch.Tensor):
    """Row-major E4M3 bytes [rows, K/16] -> the flat 256-k panel layout (K % 256 == 0)."""
    rows, nb = s_rows.shape
    return _panels("nvfp4_scales_to_panels", s_rows, rows, 16 * nb, 16, True)


def nvfp4_scales_to_rows(s: torch.Tensor, rows: int, K: int):
    """Panel-layout E4M3 bytes (flat, rows*K/16) -> row-major [rows, K/16]."""
    return _panels("nvfp4_scales_to_rows", s, rows, K, 16, False)
