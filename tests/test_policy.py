"""The activation group-size policy: the selection rule (CPU) and one run on
the device over a small heavy-tailed layer (GPU)."""
import numpy as np
import pytest

from w4a4_quantized_gemm_quantize_amd import synth
from w4a4_quantized_gemm_quantize_amd.policy import select


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
