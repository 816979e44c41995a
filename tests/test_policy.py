"""The granularity policy: the selection rule and the rho model (CPU), and runs
on the device over a small heavy-tailed layer (GPU)."""
import numpy as np
import pytest

from w4a4_quantized_gemm_quantize_amd import synth
from w4a4_quantized_gemm_quantize_amd.policy import predict_us, rho, select

RATES = {"fp6_tflops": 7000.0, "valu_f32_tflops": 78.6}


def test_select_rule():
    t = [{"group_a": 64, "rel_err": 0.100, "gemm_us": 100.0},
         {"group_a": 128, "rel_err": 0.105, "gemm_us": 80.0},
         {"group_a": 256, "rel_err": 0.150, "gemm_us": 70.0},
         {"group_a": "K", "rel_err": 0.300, "gemm_us": 60.0}]
    assert select(t, 0.10)["group_a"] == 128      # fastest within 10 % of the best error
    assert select(t, 0.0)["group_a"] == 64        # only the most accurate
    assert select(t, 5.0)["group_a"] == "K"       # everything admissible: the fastest
    t2 = [dict(r, gemm_us=50.0) for r in t]
    assert select(t2, 5.0)["group_a"] == 64       # equal speed: the smaller error


def test_rho_model():
    """The model's terms, checked by hand for one shape and by their structure:
    g_min = 128 with per-group scales on both sides costs 2MNK at the matrix
    rate + 2 MN K/128 at the fp32 matrix rate (scale products) + 2 MN K/128 at
    the vector rate (epilogue fmas)."""
    M, N, K = 4096, 28672, 8192
    t = predict_us(M, N, K, 128, 128, RATES)
    hand = (2 * M * N * K / 7000e12 + 2 * M * N * 64 / 157.3e12 + 2 * M * N * 64 / 78.6e12) * 1e6
    assert abs(t - hand) <= 1e-9 * hand
    assert abs(rho(RATES) - 7000 / 78.6) < 1e-9
    # same g_min, same cost: coarser A groups do not help with per-group W scales
    assert predict_us(M, N, K, 512, 128, RATES) == t
    # per-channel W lets coarse A groups shorten the epilogue
    assert predict_us(M, N, K, 512, K, RATES) < predict_us(M, N, K, 256, K, RATES) < t
    # per-token A needs no scale product
    assert predict_us(M, N, K, K, 128, RATES) < t
    # a finer group doubles the epilogue; a faster vector unit (smaller rho) shrinks it
    assert predict_us(M, N, K, 64, 128, RATES) > t
    fast = dict(RATES, valu_f32_tflops=2 * RATES["valu_f32_tflops"])
    assert predict_us(M, N, K, 128, 128, fast) < t and rho(fast) < rho(RATES)


def test_select_over_pairs():
    t = [{"group_a": 128, "group_w": 128, "rel_err": 0.20, "gemm_us": 880.0},
         {"group_a": 512, "group_w": "K", "rel_err": 0.21, "gemm_us": 700.0},
         {"group_a": "K", "group_w": "K", "rel_err": 0.40, "gemm_us": 600.0}]
    assert select(t, 0.10)["group_w"] == "K" and select(t, 0.10)["group_a"] == 512
    assert select(t, 0.01)["group_a"] == 128


@pytest.mark.gpu
def test_granularity_pairs_on_device():
    """(g_a, g_w) pairs with per-channel weights: the table covers every
    nesting pair, its errors are the oracle's, and the rho model ranks per
    group count the way the device times do (fewer blocks, less time)."""
    import torch
    import oracle
    from w4a4_quantized_gemm_quantize_amd.policy import choose_granularity
    dev = torch.device("cuda:0")
    K, N = 2048, 768
    x = torch.from_numpy(synth.activations(128, K, dist="t3", seed=5)).to(dev)
    w = torch.from_numpy(synth.weights(N, K, seed=6)).to(dev)
    r = choose_granularity(x, w, tokens=2048, n_cols=256, reps=3, seed=0, rates=RATES)
    tab = {(e["group_a"], e["group_w"]): e for e in r["table"]}
    assert set(tab) == {(a, b) for a in (64, 128, 256, 512, "K") for b in (128, "K")}
    assert all(e["pred_us"] > 0 for e in tab.values())
    x16 = x.cpu().numpy()
    cols = np.sort(np.random.default_rng(0).choice(N, size=256, replace=False))
    ws16 = w.cpu().numpy()[cols]
    ref = x16.astype(np.float64) @ ws16.astype(np.float64).T
    for ga, gw in ((512, "K"), (128, 128), ("K", "K")):
        a, b = (K if ga == "K" else ga), (K if gw == "K" else gw)
        Y, _ = oracle.w4a4_gemm(*oracle.int4_quantize(x16, a), a, *oracle.int4_quantize(ws16, b), b)
        e = np.linalg.norm(Y - ref) / np.linalg.norm(ref)
        assert abs(tab[(ga, gw)]["rel_err"] - e) <= 1e-4 * e, (ga, gw)
    # per-channel W: the model's and the device's order agree between the finest
    # and the coarsest activation group
    assert tab[(64, "K")]["pred_us"] > tab[("K", "K")]["pred_us"]
    assert tab[(64, "K")]["gemm_us"] > tab[("K", "K")]["gemm_us"]


@pytest.mark.gpu
def test_policy_on_device():
    import torch
    from w4a4_quantized_gemm_quantize_amd.policy import choose_group_a
    dev = torch.device("cuda:0")
    K, N = 2048, 768
    x = torch.from_numpy(synth.activations(128, K, dist="t3", seed=3)).to(dev)
    w = torch.from_numpy(synth.weights(N, K, seed=4)).to(dev)
    r = choose_group_a(x, w, tokens=512, n_cols=256, reps=3, seed=0)
    tab = {e["group_a"]: e for e in r["table"]}
    assert set(tab) == {64, 128, 256, 512, "K"}
    assert all(e["gemm_us"] > 0 for e in tab.values())
    # the error the policy measures on the device is the oracle's, up to the
    # GEMM's fp32 rounding (same column sample: seed 0)
    import oracle
    x16 = x.cpu().numpy()
    cols = np.sort(np.random.default_rng(0).choice(N, size=256, replace=False))
    ws16 = w.cpu().numpy()[cols]
    ref = x16.astype(np.float64) @ ws16.astype(np.float64).T
    qw, sw = oracle.int4_quantize(ws16, 128)
    errs = []
    for g in (64, 128, 256, 512, "K"):
        ga = K if g == "K" else g
        Y, _ = oracle.w4a4_gemm(*oracle.int4_quantize(x16, ga), ga, qw, sw, 128)
        e = np.linalg.norm(Y - ref) / np.linalg.norm(ref)
        assert abs(tab[g]["rel_err"] - e) <= 1e-4 * e, (g, tab[g]["rel_err"], e)
        errs.append(e)
    # finer groups isolate the outlier channels: the error grows with the group
    assert all(a < b for a, b in zip(errs, errs[1:]))
    best = min(e["rel_err"] for e in tab.values())
    assert tab[r["group_a"]]["rel_err"] <= 1.10 * best + 1e-12
