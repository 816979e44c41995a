"""The seeded input generator (CPU only): determinism, row-subset regeneration,
and the shape of the distributions it promises."""
import numpy as np

from w4a4_quantized_gemm_quantize_amd import synth


def test_deterministic_and_row_subsets():
    a = synth.activations(40, 512, dist="t3", seed=0)
    b = synth.activations(40, 512, dist="t3", seed=0)
    assert a.dtype == np.float16 and a.shape == (40, 512)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    rows = [3, 17, 39]
    assert np.array_equal(synth.activations(40, 512, dist="t3", seed=0, rows=rows), a[rows])
    w = synth.weights(30, 256, seed=1)
    assert np.array_equal(synth.weights(30, 256, seed=1, rows=[29, 0]), w[[29, 0]])
    assert not np.array_equal(synth.activations(40, 512, dist="t3", seed=1), a)


def test_outlier_channels():
    K = 4096
    ch = synth.outlier_channels(K, synth.default_outlier_count(K), seed=0)
    assert ch.size == 41 and np.unique(ch).size == 41
    x = synth.activations(256, K, dist="t3", seed=0).astype(np.float64)
    med = np.median(np.abs(x), axis=0)
    others = np.setdiff1d(np.arange(K), ch)
    assert np.median(med[ch]) > 20 * np.median(med[others])
    x1 = synth.activations(16, 256, dist="normal", seed=0).astype(np.float64)
    ch1 = synth.outlier_channels(256, 4, seed=0)
    assert ch1.size == 4
    assert np.abs(x1[:, ch1]).mean() > 10 * np.abs(np.delete(x1, ch1, axis=1)).mean()


def test_weight_std():
    w = synth.weights(256, 4096, seed=0).astype(np.float64)
    assert abs(w.std() - 0.02) < 5e-4 and abs(w.mean()) < 1e-4
