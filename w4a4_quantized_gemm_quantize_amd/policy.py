"""Activation group-size policy for one linear layer (APEX4 abstract, APEX4
page: mixed granularity, choosing the quantization granularity per layer from
the balance of matrix and vector work, which on this part is measured rather
than modelled).

For each candidate activation group g_a the layer is run through this
library's own kernels twice:

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


def choose_group_a(x_cal: torch.Tensor, w: torch.Tensor, group_w: int = 128, tokens: int | None = None,
                   candidates=CANDIDATES, slack: float = 0.10, n_cols: int = 512, reps: int = 10,
                   seed: int = 0):
    """Pick g_a for the linear Y = X W^T.

    x_cal: fp16 [m, K] calibration activations on the device; w: fp16 [N, K]
    weights on the device; tokens: the production token count (default m).
    Returns ``{"group_a": g, "table": [{"group_a", "rel_err", "gemm_us"}, ...]}``.
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
    wq_s, ws_s = ops.w4a4_pack_weight(w_s, group_w)
    wq, ws = ops.w4a4_pack_weight(w, group_w)
    x_big = x_cal if tokens == m else x_cal[torch.arange(tokens, device=x_cal.device) % m].contiguous()
    table = []
    for c in candidates:
        g = K if c == "K" else int(c)
        if K % g or (g != K and (g & (g - 1))):
            continue
        xq, xs = ops.w4a4_quantize_act(x_cal, g)
        y = ops.w4a4_gemm(xq, xs, g, wq_s, ws_s, group_w).cpu().numpy().astype(np.float64)
        err = float(np.linalg.norm(y - ref) / ref_norm) if ref_norm > 0 else 0.0
        bq, bs = ops.w4a4_quantize_act(x_big, g)
        us = _time_gemm(bq, bs, g, wq, ws, group_w, reps)
        table.append({"group_a": "K" if g == K else g, "rel_err": err, "gemm_us": us})
    choice = select(table, slack)
    return {"group_a": choice["group_a"], "table": table}


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
    for name in (f"{args.workload}_w13", f"{args.workload}_w2"):
        wl = synth.WORKLOADS[name]
        K, N = wl["K"], wl["N"]
        x = torch.from_numpy(synth.activations(args.cal, K, dist=wl["dist"], seed=1)).to(dev)
        w = torch.from_numpy(synth.weights(N, K, seed=0)).to(dev)
        r = choose_group_a(x, w, tokens=args.tokens, slack=args.slack)
        print(json.dumps({"linear": name, "K": K, "N": N, "tokens": args.tokens, **r}), flush=True)


if __name__ == "__main__":
    _main()
