"""Granularity policy for one linear layer (APEX4 abstract, APEX4 page:
rho-aware granularity adaptation, a mixed-granularity mode chosen from the
balance of matrix and vector work, rho being the matrix-unit : vector-unit
throughput ratio).

The group epilogue costs one vector fma per output per block of
g_min = min(g_a, g_w) along K, against 2 g_min matrix operations, so its share
of the time grows with rho / g_min. With per-group weight scales (g_w = 128)
every g_a >= 128 leaves g_min = 128; coarser activation groups only shorten
the epilogue when the weights go per output channel (g_w = K), which is the
mixed-granularity lever. The candidates are therefore (g_a, g_w) pairs with
g_a in {64, 128, 256, 512, K} and g_w in {group_w, K}.

``predict_us`` is the rho model: matrix time (the partials at the FP6 matrix
rate plus, unless g_a = K, the rank-1 scale products at the fp32 matrix rate)
plus vector time (one fma per output per block at the vector unit's fp32 fma
rate), added rather than overlapped (on this part a wave does not run its
vector work under its own matrix instructions). The rates are this GPU's,
measured by the probe kernels (``peaks.measure_peaks``), so rho is measured,
not assumed. The model ranks the candidates; the policy still times them.

For each candidate the layer is run through this library's own kernels twice:

* accuracy: the calibration activations ``x_cal`` [m, K] are quantized with
  g_a and multiplied with W (weight group ``group_w``) for a sample of output
  columns; the relative Frobenius error of Y is taken against the float64
  product of the fp16 inputs (a plain host matmul of the calibration sample,
  the reference the method approximates);
* speed: the GEMM is timed at the production shape [tokens, K] x [N, K] with
  HIP events on the launch stream (back to back behind a spin kernel).

The policy returns the fastest candidate whose error is within ``1 + slack``
of the smallest error seen. Group sizes that do not divide K are skipped. This
is a tuning step run once per layer, outside the hot path.
"""
from __future__ import annotations

import numpy as np
import torch

from . import ops

CANDIDATES = (64, 128, 256, 512, "K")
WEIGHT_CANDIDATES = (128, "K")

# fp32 matrix rate of the rank-1 scale products (v_mfma_f32_32x32x1_2b_f32);
# the data sheet's dense fp32 matrix figure, TFLOP/s
F32_MATRIX_TFLOPS = 157.3


def rho(rates) -> float:
    """This GPU's matrix : vector throughput ratio: FP6 matrix ops (the
    partials' instruction) per fp32 vector op."""
    return rates["fp6_tflops"] / rates["valu_f32_tflops"]


def predict_us(M: int, N: int, K: int, ga: int, gw: int, rates) -> float:
    """rho model of the W4A4 GEMM time (microseconds) for groups (ga, gw) with
    the rates (TFLOP/s) of ``peaks.measure_peaks``: matrix time plus vector
    time, see the module docstring."""
    gmin = min(ga, gw)
    blocks = M * N * (K // gmin)                   # output x group pairs
    t_matrix = 2.0 * M * N * K / (rates["fp6_tflops"] * 1e12)
    if ga != K:                                    # per-token A scales need no scale product
        t_matrix += 2.0 * blocks / (F32_MATRIX_TFLOPS * 1e12)
    t_vector = 2.0 * blocks / (rates["valu_f32_tflops"] * 1e12)
    return (t_matrix + t_vector) * 1e6


def select(table, slack: float):
    """The fastest entry whose ``rel_err`` is within ``(1 + slack)`` of the
    smallest ``rel_err`` (ties by speed go to the smaller error)."""
    best = min(r["rel_err"] for r in table)
    ok = [r for r in table if r["rel_err"] <= (1.0 + slack) * best]
    return min(ok, key=lambda r: (r["gemm_us"], r["rel_err"]))


def _time_gemm(xq, xs, ga, wq, ws, gw, reps):
    y = torch.empty((xq.shape[0], wq.shape[0]), dtype=torch.float32, device=xq.device)
    for _ in range(2):
        ops.w4a4_gemm(xq, xs, ga, wq, ws, gw, out=y)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(2_000_000)
    e0.record()
    for _ in range(reps):
        ops.w4a4_gemm(xq, xs, ga, wq, ws, gw, out=y)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def choose_granularity(x_cal: torch.Tensor, w: torch.Tensor, tokens: int | None = None,
                       candidates=CANDIDATES, weight_candidates=WEIGHT_CANDIDATES, slack: float = 0.10,
                       n_cols: int = 512, reps: int = 10, seed: int = 0, rates=None):
    """Pick (g_a, g_w) for the linear Y = X W^T.

    x_cal: fp16 [m, K] calibration activations on the device; w: fp16 [N, K]
    weights on the device; tokens: the production token count (default m);
    rates: measured peaks (``peaks.measure_peaks``) for the rho model, or None.
    Returns ``{"group_a": ga, "group_w": gw, "rho": r, "table": [{"group_a",
    "group_w", "rel_err", "gemm_us", "pred_us"}, ...]}`` ("K" marks a group of
    the whole row: per token for A, per output channel for W).
    """
    if x_cal.dtype != torch.float16 or w.dtype != torch.float16:
        raise TypeError("x_cal and w must be fp16")
    m, K = x_cal.shape
    N = w.shape[0]
    tokens = tokens or m
    cols = np.sort(np.random.default_rng(seed).choice(N, size=min(n_cols, N), replace=False))
    w_s = w[torch.from_numpy(cols).to(w.device)].contiguous()
    ref = x_cal.cpu().numpy().astype(np.float64) @ w_s.cpu().numpy().astype(np.float64).T
    ref_norm = np.linalg.norm(ref)
    x_big = x_cal if tokens == m else x_cal[torch.arange(tokens, device=x_cal.device) % m].contiguous()

    def group(c):
        g = K if c == "K" else int(c)
        return g if K % g == 0 and (g == K or (g & (g - 1)) == 0) else None

    table = []
    for cw in weight_candidates:
        gw = group(cw)
        if gw is None:
            continue
        wq_s, ws_s = ops.w4a4_pack_weight(w_s, gw)
        wq, ws = ops.w4a4_pack_weight(w, gw)
        for ca in candidates:
            ga = group(ca)
            if ga is None or max(ga, gw) % min(ga, gw):
                continue
            xq, xs = ops.w4a4_quantize_act(x_cal, ga)
            y = ops.w4a4_gemm(xq, xs, ga, wq_s, ws_s, gw).cpu().numpy().astype(np.float64)
            err = float(np.linalg.norm(y - ref) / ref_norm) if ref_norm > 0 else 0.0
            bq, bs = ops.w4a4_quantize_act(x_big, ga)
            us = _time_gemm(bq, bs, ga, wq, ws, gw, reps)
            table.append({"group_a": "K" if ga == K else ga, "group_w": "K" if gw == K else gw, "rel_err": err,
                          "gemm_us": us,
                          "pred_us": predict_us(tokens, N, K, ga, gw, rates) if rates else None})
    choice = select(table, slack)
    return {"group_a": choice["group_a"], "group_w": choice["group_w"],
            "rho": rho(rates) if rates else None, "table": table}


def choose_group_a(x_cal: torch.Tensor, w: torch.Tensor, group_w: int = 128, tokens: int | None = None,
                   candidates=CANDIDATES, slack: float = 0.10, n_cols: int = 512, reps: int = 10,
                   seed: int = 0):
    """Pick g_a alone for a fixed weight group (the table of
    :func:`choose_granularity` restricted to g_w = group_w)."""
    r = choose_granularity(x_cal, w, tokens, candidates, (group_w,), slack, n_cols, reps, seed)
    return {"group_a": r["group_a"], "table": [{k: e[k] for k in ("group_a", "rel_err", "gemm_us")}
                                                for e in r["table"]]}


def _main():
    """Run the policy on the FFN linears of a named workload with synthetic
    calibration activations (seeded, heavy-tailed with outlier channels) and
    synthetic weights; print one JSON line per linear."""
    import argparse
    import json

    from . import synth
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="llama2_70b", choices=["llama2_7b", "llama2_70b"])
    ap.add_argument("--tokens", type=int, default=4096)
    ap.add_argument("--cal", type=int, default=256, help="calibration tokens")
    ap.add_argument("--slack", type=float, default=0.10)
    args = ap.parse_args()
    dev = torch.device("cuda:0")
    from .peaks import measure_peaks
    rates = measure_peaks()
    for name in (f"{args.workload}_w13", f"{args.workload}_w2"):
        wl = synth.WORKLOADS[name]
        K, N = wl["K"], wl["N"]
        x = torch.from_numpy(synth.activations(args.cal, K, dist=wl["dist"], seed=1)).to(dev)
        w = torch.from_numpy(synth.weights(N, K, seed=0)).to(dev)
        r = choose_granularity(x, w, tokens=args.tokens, slack=args.slack, rates=rates)
        print(json.dumps({"linear": name, "K": K, "N": N, "tokens": args.tokens, **r}), flush=True)


if __name__ == "__main__":
    _main()
