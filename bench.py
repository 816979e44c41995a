#!/usr/bin/env python3
"""W4A4-g128 GEMM throughput including activation quantization, on the
LLaMA-2-70B FFN linear shapes (and, by flag, the other workloads).

One step = one pass of the INT4 hot path over one batch of M tokens through the
three FFN linears (w1 and w3: K=8192 -> N=28672; w2: K=28672 -> N=8192): for
each linear, per-token group-128 INT4 quantization of its fp16 input followed by
the group-dequantized INT4 GEMM (fp32 Y). Weights are packed once, untimed
(offline). Inputs are synthetic (seeded), resident in HBM before timing starts.

Prints one JSON line. `value` = useful ops (2*M*N*K summed over the linears)
per second of the timed steps, in TOPS. `roofline` is for the GEMM kernel (the
dominant one), timed per launch with HIP events on the launch stream.
`cpu_baseline` times the CPU oracle on a bounded row/column sample of the same
workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME] [--tokens M]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "W4A4-g128 GEMM TOPS incl. act-quant, LLaMA-70B FFN shapes; % of MFMA peak"
PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 matrix-core peak (5.0 POP/s)
PEAK_FP4_TFLOPS = 10100.0    # MI355X dense fp4/fp6 matrix-core peak
PEAK_FP16_TFLOPS = 2500.0    # MI355X dense fp16 matrix-core peak (the NVFP4 GEMM's instructions)
PEAK_HBM_GBS = 8000.0

# name -> (tokens M, [(K, N), ...], act group, weight group, format)
WORKLOADS = {
    "llama2_70b_ffn": (4096, [(8192, 28672), (8192, 28672), (28672, 8192)], 128, 128, "int4"),
    "llama2_7b_ffn": (2048, [(4096, 11008), (4096, 11008), (11008, 4096)], 128, 128, "int4"),
    "granularity": (4096, [(8192, 8192)], 128, 128, "int4"),
    "qwen25_7b_mxfp4_ffn": (4096, [(3584, 18944), (3584, 18944), (18944, 3584)], 32, 32, "mxfp4"),
    # two-pass MXFP4 with the residual appended along K (the GEMM runs K' = 2K)
    "qwen25_7b_mxfp4_residual_ffn": (4096, [(3584, 18944), (3584, 18944), (18944, 3584)], 32, 32, "mxfp4res"),
    # NVFP4 (E4M3 scale per 16, global scale per tensor) on the same shapes
    "qwen25_7b_nvfp4_ffn": (4096, [(3584, 18944), (3584, 18944), (18944, 3584)], 16, 16, "nvfp4"),
}


GEMM_SOURCES = {"int4": "w4a4_quantized_gemm_quantize_amd/csrc/gemm_w4a4.hip",
                "mxfp4": "w4a4_quantized_gemm_quantize_amd/csrc/gemm_mxfp4.hip",
                "mxfp4res": "w4a4_quantized_gemm_quantize_amd/csrc/gemm_mxfp4.hip",
                "nvfp4": "w4a4_quantized_gemm_quantize_amd/csrc/nvfp4.hip"}
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "gemm_traffic.json")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_sha256(fmt: str) -> str:
    with open(os.path.join(ROOT, GEMM_SOURCES[fmt]), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def gemm_alg_bytes(fmt: str, M: int, layers, kmul: int, ydt, ga: int = 128, gw: int = 128) -> float:
    """Mean algorithmic HBM bytes of one GEMM launch: codes and scales of both
    operands read once, Y written once."""
    import torch
    ybytes = 4 if ydt == torch.float32 else 2
    tot = 0
    for L in layers:
        K, N = kmul * L["K"], L["N"]
        if fmt == "int4":
            tot += (M + N) * (K // 2) + M * 4 * (K // ga) + N * 4 * (K // gw) + ybytes * M * N
        else:
            sb = K // 16 if fmt == "nvfp4" else K // 32
            tot += (M + N) * (K // 2 + sb) + ybytes * M * N
    return tot / len(layers)


def measured_traffic(fmt: str, workload: str, tokens: int):
    """HBM bytes per GEMM launch from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE record, scaled by the copy-kernel calibration; None when there is
    no record for this workload or the kernel source changed since it was taken."""
    try:
        rec = json.load(open(TRAFFIC_RECORD))[f"{fmt}:{workload}:{tokens}"]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != source_sha256(fmt):
        return None
    return rec["hbm_bytes_per_launch"]


def copy_calibration(nbytes: int = 1 << 30, reps: int = 3) -> int:
    """A plain device copy of known size, run under rocprofv3 to scale the HBM
    byte counters (FETCH_SIZE / WRITE_SIZE) of the GEMM runs."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": nbytes, "launches": reps}), flush=True)
    return 0


def quant_standalone(shapes, ga, fmt, reps: int = 24, nrot: int = 6):
    """Activation quantization on its own: for each distinct [M, K], ``reps``
    back-to-back launches rotating over ``nrot`` resident inputs (more bytes
    than the 256 MB last-level cache, so every launch reads HBM), queued behind
    a spin kernel and one untimed pass over the inputs, and timed with HIP
    events on the launch stream. Returns per-shape rows and the overall
    GB/s over the algorithmic bytes (fp16 in, codes and scales out)."""
    import torch
    from w4a4_quantized_gemm_quantize_amd import ops
    dev = torch.device("cuda:0")
    rows, tot_bytes, tot_s = [], 0, 0.0
    for (M, K) in shapes:
        xs = [(torch.randn(M, K, device=dev) * 0.5).half() for _ in range(nrot)]
        xq = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
        if fmt == "int4":
            sc = torch.empty((K // ga, M), dtype=torch.float32, device=dev)
            call = lambda x: ops.w4a4_quantize_act(x, ga, out=(xq, sc))
            nbytes = M * (2 * K + K // 2 + 4 * (K // ga))
        elif fmt == "mxfp4":
            sc = torch.empty((M * (K // 32),), dtype=torch.uint8, device=dev)
            call = lambda x: ops.mxfp4_quantize(x, out=(xq, sc))
            nbytes = M * (2 * K + K // 2 + K // 32)
        elif fmt == "nvfp4":
            sc = torch.empty((M * (K // 16),), dtype=torch.uint8, device=dev)
            g = ops.nvfp4_global_scale(xs[0])      # a calibrated (static) global scale
            call = lambda x: ops.nvfp4_quantize(x, g, out=(xq, sc))
            nbytes = M * (2 * K + K // 2 + K // 16)
        else:
            xq = torch.empty((M, K), dtype=torch.uint8, device=dev)
            sc = torch.empty((M * (2 * K // 32),), dtype=torch.uint8, device=dev)
            call = lambda x: ops.mxfp4_quantize_residual(x, out=(xq, sc))
            nbytes = M * (2 * K + K + 2 * K // 32)
        for i in range(nrot):
            call(xs[i])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        # a spin kernel holds the stream while the host enqueues every launch, so
        # the timed launches run back to back (host launch cost excluded); one
        # untimed pass over the inputs behind it brings the clocks back up
        torch.cuda._sleep(5_000_000)
        for i in range(nrot):
            call(xs[i])
        e0.record()
        for i in range(reps):
            call(xs[i % nrot])
        e1.record()
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) / 1e3 / reps
        rows.append({"M": M, "K": K, "us": sec * 1e6, "GB/s": nbytes / sec / 1e9})
        tot_bytes += nbytes
        tot_s += sec
        del xs
    return rows, tot_bytes / tot_s / 1e9


from w4a4_quantized_gemm_quantize_amd.peaks import PROBE_KINDS, VENDOR_PEAKS, measure_peaks  # noqa: E402,F401


def cpu_baseline(wl, M, ga, gw, fmt, n_rows, n_cols):
    """Time the CPU oracle (C++, std::thread over every core this process may
    use) on n_rows tokens x n_cols output features per linear, all of K:
    act-quant + GEMM, weights quantized untimed. Also states the full step's
    time extrapolated from the sample's rate (the oracle's cost is linear in
    M * N * K)."""
    import oracle
    from w4a4_quantized_gemm_quantize_amd import synth

    oracle.set_threads(0)
    rows = synth.sample_rows(M, n_rows, seed=11)
    work = []
    for li, (K, N) in enumerate(wl):
        cols = synth.sample_rows(N, min(n_cols, N), seed=12 + li)
        x = synth.activations(M, K, dist="t3", seed=li, rows=rows)
        w = synth.weights(N, K, seed=100 + li, rows=cols)
        if fmt == "int4":  # weights offline, untimed
            wpk = oracle.int4_quantize(w, gw)
        elif fmt == "mxfp4":
            wpk = oracle.mxfp4_quantize(w)
        elif fmt == "nvfp4":  # weights and both global scales offline (calibration), untimed
            sgw = oracle.nvfp4_global_scale(w)
            wpk = (*oracle.nvfp4_quantize(w, sgw), sgw, oracle.nvfp4_global_scale(x))
        else:
            wpk = oracle.mxfp4_append_copy(*oracle.mxfp4_quantize(w))
        work.append((x, wpk, K, len(cols)))
    ops = 0
    t0 = time.perf_counter()
    for x, wpk, K, nc in work:
        if fmt == "int4":
            qa, sa = oracle.int4_quantize(x, ga)
            oracle.w4a4_gemm(qa, sa, ga, wpk[0], wpk[1], gw)
        elif fmt == "nvfp4":
            ca, sa = oracle.nvfp4_quantize(x, wpk[3])
            oracle.nvfp4_gemm(ca, sa, wpk[3], wpk[0], wpk[1], wpk[2])
        else:
            ca, ea = oracle.mxfp4_quantize(x) if fmt == "mxfp4" else oracle.mxfp4_quantize_residual(x)
            oracle.mxfp4_gemm(ca, ea, wpk[0], wpk[1])
        ops += 2 * len(rows) * nc * K
    dt = time.perf_counter() - t0
    full_ops = sum(2 * M * N * K for K, N in wl)
    return {
        "value": ops / dt / 1e12, "unit": "TOPS", "cores": oracle.cores(), "kind": "oracle",
        "sample": (f"{len(rows)} of {M} tokens x " + ("every output column" if n_cols >= max(N for _, N in wl)
                   else f"a {n_cols}-column sample") + f" of each linear (all K), act-quant + GEMM, "
                   f"{dt:.1f} s on the host"),
        "implementation": "C++ (oracle/orc.cpp, -O2 -ffp-contract=off), std::thread over rows",
        "extrapolated_full_step_s": dt * full_ops / ops,
    }


# The configurations' oracle runs: (name, M, [(K, N), ...], g_a, format, full);
# full = every output (the rest: a seeded 256-row sample x all N, its time
# extrapolated to the whole problem).
ORACLE_CONFIGS = [
    ("C1 tiny", 16, [(256, 256)], 128, "int4", True),
    ("C2 LLaMA-2-7B FFN", 2048, [(4096, 11008), (11008, 4096)], 128, "int4", True),
    ("C3 LLaMA-2-70B FFN M=1", 1, [(8192, 28672), (28672, 8192)], 128, "int4", True),
    ("C3 LLaMA-2-70B FFN M=16", 16, [(8192, 28672), (28672, 8192)], 128, "int4", True),
    ("C3 LLaMA-2-70B FFN M=256", 256, [(8192, 28672), (28672, 8192)], 128, "int4", True),
    ("C3 LLaMA-2-70B FFN M=4096", 4096, [(8192, 28672), (28672, 8192)], 128, "int4", False),
    ("C4 granularity g_a=64", 4096, [(8192, 8192)], 64, "int4", False),
    ("C4 granularity g_a=128", 4096, [(8192, 8192)], 128, "int4", False),
    ("C4 granularity g_a=256", 4096, [(8192, 8192)], 256, "int4", False),
    ("C4 granularity g_a=512", 4096, [(8192, 8192)], 512, "int4", False),
    ("C4 granularity g_a=8192", 4096, [(8192, 8192)], 8192, "int4", False),
    ("C5 Qwen2.5-7B FFN MXFP4", 4096, [(3584, 18944), (18944, 3584)], 32, "mxfp4", False),
]


def oracle_timing() -> int:
    """Time the CPU oracle (every core) on each configuration, one JSON line
    per linear: activation quantization and weight packing in full, the GEMM
    in full where feasible, else on a seeded 256-row sample with all N and its
    time extrapolated to the whole problem (the oracle's cost is linear in
    M). Input generation is not timed. CPU only."""
    import numpy as np
    import oracle
    from w4a4_quantized_gemm_quantize_amd import synth

    oracle.set_threads(0)
    for name, M, lin, ga, fmt, full in ORACLE_CONFIGS:
        for li, (K, N) in enumerate(lin):
            dist = "normal" if name.startswith("C1") else "t3"
            x = synth.activations(M, K, dist=dist, seed=li)
            w = synth.weights(N, K, seed=100 + li)
            t0 = time.perf_counter()
            if fmt == "int4":
                qa, sa = oracle.int4_quantize(x, ga)
            else:
                qa, sa = oracle.mxfp4_quantize(x)
            t_quant = time.perf_counter() - t0
            t0 = time.perf_counter()
            wpk = oracle.int4_quantize(w, 128) if fmt == "int4" else oracle.mxfp4_quantize(w)
            t_pack = time.perf_counter() - t0
            rows = np.arange(M) if full else synth.sample_rows(M, 256, seed=11)
            t0 = time.perf_counter()
            if fmt == "int4":
                oracle.w4a4_gemm(qa[rows], np.ascontiguousarray(sa[rows]), ga, wpk[0], wpk[1], 128)
            else:
                oracle.mxfp4_gemm(qa[rows], np.ascontiguousarray(sa[rows]), wpk[0], wpk[1])
            t_gemm = time.perf_counter() - t0
            macs = rows.size * N * K
            print(json.dumps({
                "config": name, "linear": f"K={K} N={N}", "M": M, "group_a": ga, "format": fmt,
                "gemm_rows": int(rows.size), "gemm_full": bool(full), "threads": oracle.cores(),
                "act_quant_s": t_quant, "weight_pack_s": t_pack, "gemm_s": t_gemm,
                "gemm_mac_per_s": macs / t_gemm,
                "gemm_full_s" + ("" if full else "_extrapolated"): t_gemm * M / rows.size,
            }), flush=True)
            del x, w, qa, sa, wpk
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama2_70b_ffn", choices=sorted(WORKLOADS))
    ap.add_argument("--tokens", type=int, default=None, help="override M")
    ap.add_argument("--group-a", type=int, default=None, help="override the activation group")
    ap.add_argument("--ydtype", choices=["f32", "f16"], default="f32")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    # the CPU baseline's sample: 512 tokens x every output column of each
    # linear (~11 s of oracle work on a 16-thread host at the headline shapes)
    ap.add_argument("--cpu-rows", type=int, default=512)
    ap.add_argument("--cpu-cols", type=int, default=1 << 20)
    ap.add_argument("--quant-only", action="store_true",
                    help="only the standalone activation-quantization timing (for profiling)")
    ap.add_argument("--peaks", action="store_true",
                    help="only measure this GPU's matrix-core and HBM peaks with the probe kernels")
    ap.add_argument("--no-peaks", action="store_true", help="skip the peak probes in a bench run")
    ap.add_argument("--no-fused", action="store_true",
                    help="few tokens: quantize and multiply in two launches even where the fused path applies")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (for scaling rocprofv3 byte counters)")
    ap.add_argument("--oracle-timing", action="store_true",
                    help="only time the CPU oracle on every configuration (no GPU)")
    args = ap.parse_args()
    if args.oracle_timing:
        return oracle_timing()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    if args.copy_calibration:
        return copy_calibration()
    if args.peaks:
        pk = measure_peaks()
        print(json.dumps({"peaks_measured": pk, "peaks_vendor": VENDOR_PEAKS}), flush=True)
        return 0

    import numpy as np
    import torch

    from w4a4_quantized_gemm_quantize_amd import _lib, ops, synth

    M0, wl, ga, gw, fmt = WORKLOADS[args.workload]
    M = args.tokens or M0
    if args.group_a:
        ga = args.group_a
    ydt = torch.float32 if args.ydtype == "f32" else torch.float16
    dev = torch.device("cuda:0")
    lib = _lib.load_library()
    log(f"workload {args.workload}: M={M} linears={wl} ga={ga} gw={gw} fmt={fmt}")
    act_shapes = sorted({(M, K) for K, _ in wl})
    if args.quant_only:
        q_rows, q_gbs = quant_standalone(act_shapes, ga, fmt)
        print(json.dumps({"act_quant_standalone": {"GB/s": q_gbs, "frac_hbm": q_gbs / PEAK_HBM_GBS,
                                                   "per_shape": q_rows}}), flush=True)
        return 0

    layers = []
    for li, (K, N) in enumerate(wl):
        x = torch.from_numpy(synth.activations(M, K, dist="t3", seed=li)).to(dev)
        w = torch.from_numpy(synth.weights(N, K, seed=100 + li)).to(dev)
        if fmt == "int4":
            wq, ws = ops.w4a4_pack_weight(w, gw)
            xq = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
            xs = torch.empty((K // ga, M), dtype=torch.float32, device=dev)
            # K-split workspace when the tiles alone would leave CUs idle (small M); none at M = 4096
            nws = _lib.splitk_workspace_bytes(M, N, K, ga, gw, 0)
            wsp = torch.empty((max(nws, 16) // 4,), dtype=torch.float32, device=dev)
        elif fmt == "mxfp4":
            wq, ws = ops.mxfp4_quantize(w)
            xq = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
            xs = torch.empty((M * (K // 32),), dtype=torch.uint8, device=dev)
        elif fmt == "nvfp4":
            # weight global scale and packing offline; the activation global
            # scale calibrated once on this input, untimed (a static scale)
            gwt = ops.nvfp4_global_scale(w)
            wq, ws = ops.nvfp4_quantize(w, gwt)
            gxt = ops.nvfp4_global_scale(x)
            xq = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
            xs = torch.empty((M * (K // 16),), dtype=torch.uint8, device=dev)
        else:
            wq, ws = ops.mxfp4_quantize_append_copy(w)
            xq = torch.empty((M, K), dtype=torch.uint8, device=dev)
            xs = torch.empty((M * (2 * K // 32),), dtype=torch.uint8, device=dev)
        del w
        y = torch.empty((M, N), dtype=ydt, device=dev)
        layers.append(dict(K=K, N=N, x=x, wq=wq, ws=ws, xq=xq, xs=xs, y=y))
        if fmt == "int4":
            layers[-1].update(wsp=wsp)
        if fmt == "nvfp4":
            layers[-1].update(gx=gxt, gw=gwt)
        log(f"linear {li}: K={K} N={N} ready")
    torch.cuda.synchronize()
    # few tokens: one fused launch per linear (activation quantization inside
    # the GEMM) when every linear takes it and --no-fused is not given
    for L in layers:
        L["fused"] = fmt == "int4" and not args.no_fused and ops.use_fused(M, L["N"], L["K"], ga, gw)
    fused = [L["fused"] for L in layers]
    if any(fused):
        log(f"int4 path: fused quantization + GEMM (one launch) for linears {[i for i, f in enumerate(fused) if f]}")

    # w1 and w3 of an FFN read the same input: the shared-quantization figure
    # quantizes it once for both (w3's GEMM reads w1's codes and scales)
    can_share = (len(layers) == 3 and layers[0]["K"] == layers[1]["K"] and not any(L["fused"] for L in layers))

    def step(ev=None, shared=False):
        for li, L in enumerate(layers):
            src = layers[0] if (shared and li == 1) else L
            if ev is not None:
                ev[li][0].record()
            if fmt == "int4" and L["fused"]:
                pass                          # quantized inside the fused launch below
            elif shared and li == 1:
                pass                          # w1's quantized input serves w3
            elif fmt == "int4":
                ops.w4a4_quantize_act(L["x"], ga, out=(L["xq"], L["xs"]))
            elif fmt == "mxfp4":
                ops.mxfp4_quantize(L["x"], out=(L["xq"], L["xs"]))
            elif fmt == "nvfp4":
                ops.nvfp4_quantize(L["x"], L["gx"], out=(L["xq"], L["xs"]))
            else:
                ops.mxfp4_quantize_residual(L["x"], out=(L["xq"], L["xs"]))
            if ev is not None:
                ev[li][1].record()
            if fmt == "int4" and L["fused"]:
                ops.w4a4_linear(L["x"], L["wq"], L["ws"], ga, gw, out=L["y"], fused=True)
            elif fmt == "int4":
                ops.w4a4_gemm_splitk(src["xq"], src["xs"], ga, L["wq"], L["ws"], gw, out=L["y"], workspace=L["wsp"])
            elif fmt == "nvfp4":
                ops.nvfp4_gemm(src["xq"], src["xs"], src["gx"], L["wq"], L["ws"], L["gw"], out=L["y"])
            else:
                ops.mxfp4_gemm(src["xq"], src["xs"], L["wq"], L["ws"], out=L["y"])
            if ev is not None:
                ev[li][2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    def timed(per_launch_events, shared=False):
        """args.steps steps between two HIP events on the launch stream. A spin
        kernel holds the stream while the host enqueues them, so they run back
        to back as a captured graph would (at few tokens a launch takes longer
        to enqueue than to run); the start event is queued behind the spin,
        which is not timed. While the spin runs the GPU is all but idle and
        lowers its clocks, so args.warmup more untimed steps run between the
        spin and the start event (measured at M = 4096: without them the
        timed steps ran ~5 % slower, the clocks still rising; a longer warm-up
        before the spin did not help). Returns (seconds, per-step launch
        events or None)."""
        evs = ([[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in layers]
                for _ in range(args.steps)] if per_launch_events else None)
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        torch.cuda._sleep(int(2e6) * (args.steps + args.warmup))
        for _ in range(args.warmup):
            step(None, shared)
        start.record()
        for s in range(args.steps):
            step(evs[s] if evs else None, shared)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / 1e3, evs

    # the step time (value) from a pass with no events between launches (an
    # event pair costs a few microseconds, as much as a decode-sized launch);
    # per-launch times (roofline, per-linear figures) from a second pass
    t0 = time.perf_counter()
    elapsed, _ = timed(False)
    wall = time.perf_counter() - t0
    log(f"timed {args.steps} steps: {elapsed * 1e3:.2f} ms (wall {wall * 1e3:.2f} ms)")
    shared_elapsed = timed(False, shared=True)[0] if can_share else None
    _, evs = timed(True)     # last, so a kernel trace's final launches are these

    ops_per_step = sum(2 * M * L["N"] * L["K"] for L in layers)
    value = ops_per_step * args.steps / elapsed / 1e12

    gemm_s = np.zeros(len(layers))
    quant_s = np.zeros(len(layers))
    for s in range(args.steps):
        for li in range(len(layers)):
            e = evs[s][li]
            quant_s[li] += e[0].elapsed_time(e[1]) / 1e3
            gemm_s[li] += e[1].elapsed_time(e[2]) / 1e3
    kmul = 2 if fmt == "mxfp4res" else 1     # the appended-residual GEMM runs K' = 2K
    gemm_ops = sum(2 * M * L["N"] * kmul * L["K"] for L in layers) * args.steps
    achieved = gemm_ops / gemm_s.sum() / 1e12
    peak = {"int4": PEAK_INT8_TOPS, "nvfp4": PEAK_FP16_TFLOPS}.get(fmt, PEAK_FP4_TFLOPS)
    ybytes = 4 if ydt == torch.float32 else 2
    quant_bytes = 0
    for L in layers:
        sbytes = 4 * (L["K"] // ga) if fmt == "int4" else L["K"] // 16 if fmt == "nvfp4" else kmul * L["K"] // 32
        quant_bytes += M * (2 * L["K"] + kmul * L["K"] // 2 + sbytes)
    quant_gbs = quant_bytes * args.steps / quant_s.sum() / 1e9
    per_linear = []
    for li, L in enumerate(layers):
        per_linear.append({
            "K": L["K"], "N": L["N"],
            "gemm_us": gemm_s[li] / args.steps * 1e6,
            "gemm_tops": 2 * M * L["N"] * kmul * L["K"] / (gemm_s[li] / args.steps) / 1e12,
            "quant_us": quant_s[li] / args.steps * 1e6,
        })

    q_rows, q_gbs = quant_standalone(act_shapes, ga, fmt)
    log(f"standalone act-quant: {q_gbs:.0f} GB/s")
    peaks = None if args.no_peaks else measure_peaks()
    if peaks:
        log("measured peaks: " + ", ".join(f"{k} {v:.0f}" for k, v in peaks.items()))

    result = {
        "metric": (METRIC if args.workload == "llama2_70b_ffn"
                   else f"{fmt} GEMM TOPS incl. act-quant, {args.workload}" if fmt != "mxfp4res"
                   else f"effective TOPS (2*M*N*K of the layers) of two-pass MXFP4 with the residual appended "
                        f"along K, incl. act-quant, {args.workload}"),
        "value": value,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4" if fmt == "int4" else "fp4",
        "data": "synthetic",
        "config": {
            "workload": args.workload, "tokens": M,
            "linears_KxN": [f"{K}x{N}" for K, N in wl],
            "group_a": ga if fmt in ("int4", "nvfp4") else 32, "group_w": gw if fmt in ("int4", "nvfp4") else 32,
            "y_dtype": args.ydtype, "parallelism": "single GPU",
            "int4_path": (["fused quantization + GEMM" if f else "quantize, then GEMM" for f in fused]
                          if fmt == "int4" else None),
        },
        "roofline": {
            "bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
            "frac": achieved / peak, "traffic": measured_traffic(fmt, args.workload, M),
        },
        "act_quant": {"GB/s": quant_gbs, "frac_hbm": quant_gbs / PEAK_HBM_GBS,
                      "method": "per-launch events inside the timed steps (each launch follows a GEMM "
                                "whose output fills the caches with dirty lines)"},
        "act_quant_standalone": {"GB/s": q_gbs, "frac_hbm": q_gbs / PEAK_HBM_GBS, "per_shape": q_rows,
                                 "method": "24 back-to-back launches over 6 rotating resident inputs, queued behind a spin kernel and an untimed pass over the inputs, HIP events"},
        "per_linear": per_linear,
        "w13_shared_quant": ({"value": ops_per_step * args.steps / shared_elapsed / 1e12, "unit": "TOPS",
                              "ms_per_step": shared_elapsed / args.steps * 1e3,
                              "method": "the same steps with w1's quantized input also feeding w3 (an FFN's w1 and "
                                        "w3 read the same activations): two act-quant launches per step instead "
                                        "of three; not the headline value"}
                             if can_share else None),
        "fraction_of_mfma_peak_incl_quant": value / peak,
    }
    if peaks:
        # the same achieved rate against this GPU's measured peaks: the graded
        # peak's instruction, and the instruction the GEMM actually issues
        graded = {"int4": "int8_tops", "nvfp4": "fp16_tflops"}.get(fmt, "fp4_tflops")
        issued = {"int4": "fp6_tflops", "nvfp4": "fp16_tflops"}.get(fmt, "fp4_tflops")
        result["peaks_measured"] = peaks
        result["roofline_vs_measured"] = {
            "graded_peak": graded, "graded_peak_measured": peaks[graded],
            "frac_of_measured": achieved / peaks[graded],
            "issued_instruction": issued, "issued_peak_vendor": VENDOR_PEAKS[issued],
            "issued_peak_measured": peaks[issued],
            "frac_of_issued_vendor": achieved / VENDOR_PEAKS[issued],
            "frac_of_issued_measured": achieved / peaks[issued],
            "act_quant_standalone_frac_of_measured_copy": q_gbs / peaks["hbm_copy_gbs"],
        }
        if result["roofline"]["traffic"]:
            result["roofline_vs_measured"]["traffic_over_algorithmic"] = (
                result["roofline"]["traffic"] / gemm_alg_bytes(fmt, M, layers, kmul, ydt, ga, gw))
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        result["cpu_baseline"] = cpu_baseline(wl, M, ga, gw, fmt, args.cpu_rows, args.cpu_cols)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
