"""Seeded synthetic inputs for the W4A4 / MXFP4 linear layer.

This module draws random fp16 matrices and nothing else: it holds none of the
quantization or GEMM arithmetic, so the CPU oracle and the HIP path can both be
fed from it without sharing any of the method.

Distributions (the pages name the models whose FFN shapes are used, never their
data, so every tensor here is synthetic):

* ``"normal"``: activations ~ N(0, 1) with a few outlier input channels scaled
  up (the tiny W4A4-g128 case uses 4 channels x20).
* ``"t3"``: heavy-tailed activations 0.5 * Student-t(nu=3) with 1% of the input
  channels scaled x30. Heavy tails and channel outliers are what make per-group
  activation quantization necessary ("Depth Registers Unlock W4A4 on SwiGLU",
  abstract: outlier-dominated activation sites such as the w2 input of a
  SwiGLU block; APEX4 abstract: W4A4-g128).
* weights ~ N(0, 0.02).

Every row has its own counter-derived stream
(``SeedSequence(seed, spawn_key=(stream, row))``), so any subset of rows can be
regenerated alone and bit-identically; that is how sampled oracle checks of the
large shapes get their rows.
"""
from __future__ import annotations

import concurrent.futures
import os

import numpy as np

FP16_MAX = 65504.0

# Sub-stream ids: one per kind of tensor drawn from the same seed.
STREAM_X = 1
STREAM_W = 2
STREAM_CHANNELS = 3


def _rng(seed: int, stream: int, row: int | None = None) -> np.random.Generator:
    key = (stream,) if row is None else (stream, int(row))
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(int(seed), spawn_key=key)))


def outlier_channels(K: int, count: int, seed: int = 0) -> np.ndarray:
    """The first ``count`` entries of a seeded permutation of [0, K), sorted."""
    if count <= 0:
        return np.zeros(0, dtype=np.int64)
    perm = _rng(seed, STREAM_CHANNELS).permutation(K)
    return np.sort(perm[:count]).astype(np.int64)


def default_outlier_count(K: int) -> int:
    """1% of the input channels, rounded to nearest (at least one)."""
    return max(1, int(round(0.01 * K)))


def _to_fp16(a: np.ndarray) -> np.ndarray:
    return np.clip(a, -FP16_MAX, FP16_MAX).astype(np.float16)


def _fill_rows(out: np.ndarray, row_ids: np.ndarray, make_row) -> None:
    """out[i] = make_row(row_ids[i]); rows are independent, so large fills are
    spread over a thread pool (numpy's generators release the GIL)."""
    def fill(span):
        for i in range(*span):
            out[i] = make_row(row_ids[i])
    n = row_ids.size
    workers = min(16, os.cpu_count() or 1)
    if n < 256 or workers == 1:
        fill((0, n))
        return
    step = (n + workers * 4 - 1) // (workers * 4)
    spans = [(a, min(a + step, n)) for a in range(0, n, step)]
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        list(ex.map(fill, spans))


def activations(M: int, K: int, *, dist: str = "t3", seed: int = 0,
                n_outliers: int | None = None, outlier_scale: float | None = None,
                rows=None) -> np.ndarray:
    """fp16 activation matrix X[M, K] (or the listed ``rows`` of it).

    ``dist="normal"``: N(0,1), default 4 outlier channels x20.
    ``dist="t3"``: 0.5*t(3), default round(1% of K) outlier channels x30.
    """
    if dist == "normal":
        n_out = 4 if n_outliers is None else n_outliers
        scale = 20.0 if outlier_scale is None else outlier_scale
    elif dist == "t3":
        n_out = default_outlier_count(K) if n_outliers is None else n_outliers
        scale = 30.0 if outlier_scale is None else outlier_scale
    else:
        raise ValueError(f"unknown activation distribution {dist!r}")
    row_ids = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    if row_ids.size and (row_ids.min() < 0 or row_ids.max() >= M):
        raise IndexError("row index out of range")
    ch = outlier_channels(K, n_out, seed)
    gain = np.ones(K, dtype=np.float64)
    gain[ch] = scale
    out = np.empty((row_ids.size, K), dtype=np.float16)

    def make_row(r):
        g = _rng(seed, STREAM_X, r)
        v = g.standard_normal(K) if dist == "normal" else 0.5 * g.standard_t(3, K)
        return _to_fp16(v * gain)
    _fill_rows(out, row_ids, make_row)
    return out


def bulk_normal(M: int, K: int, *, seed: int = 0) -> np.ndarray:
    """fp16 N(0,1) matrix [M, K] from one generator, drawn in row chunks: for
    tests whose point is the row count (grid limits), where building one
    generator per row would dominate."""
    g = _rng(seed, STREAM_X, 1 << 40)
    out = np.empty((M, K), dtype=np.float16)
    step = max(1, (1 << 22) // max(K, 1))
    for r in range(0, M, step):
        n = min(step, M - r)
        out[r:r + n] = g.standard_normal((n, K), dtype=np.float32).astype(np.float16)
    return out


def weights(N: int, K: int, *, std: float = 0.02, seed: int = 0, rows=None) -> np.ndarray:
    """fp16 weight matrix W[N, K] ~ N(0, std) (or the listed ``rows`` of it)."""
    row_ids = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    if row_ids.size and (row_ids.min() < 0 or row_ids.max() >= N):
        raise IndexError("row index out of range")
    out = np.empty((row_ids.size, K), dtype=np.float16)
    _fill_rows(out, row_ids, lambda r: _to_fp16(_rng(seed, STREAM_W, r).normal(0.0, std, K)))
    return out


def sample_rows(M: int, count: int, seed: int = 0) -> np.ndarray:
    """A seeded, sorted sample of ``count`` distinct row indices of [0, M)."""
    count = min(count, M)
    return np.sort(_rng(seed, 4).choice(M, size=count, replace=False)).astype(np.int64)


# The workloads, by name. Shapes are the FFN linears of the named models; the
# data are synthetic (see module docstring).
#   (name, M, K, N, act_dist, g_a, g_w)
WORKLOADS = {
    "tiny": dict(M=16, K=256, N=256, dist="normal", g_a=128, g_w=128),
    "llama2_7b_w13": dict(M=2048, K=4096, N=11008, dist="t3", g_a=128, g_w=128),
    "llama2_7b_w2": dict(M=2048, K=11008, N=4096, dist="t3", g_a=128, g_w=128),
    "llama2_70b_w13": dict(M=4096, K=8192, N=28672, dist="t3", g_a=128, g_w=128),
    "llama2_70b_w2": dict(M=4096, K=28672, N=8192, dist="t3", g_a=128, g_w=128),
    "granularity": dict(M=4096, K=8192, N=8192, dist="t3", g_a=128, g_w=128),
    "qwen25_7b_w13": dict(M=4096, K=3584, N=18944, dist="t3", g_a=32, g_w=32),
    "qwen25_7b_w2": dict(M=4096, K=18944, N=3584, dist="t3", g_a=32, g_w=32),
}
