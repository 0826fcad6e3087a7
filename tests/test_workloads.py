"""Host-side checks of the seeded synthetic input generators."""
import numpy as np

from precision_dense_linear_amd import workloads as W


def test_deterministic_and_distinct_streams():
    a1, b1 = W.pertensor_pair(64, 48, 32, seed=3)
    a2, b2 = W.pertensor_pair(64, 48, 32, seed=3)
    assert np.array_equal(a1, a2) and np.array_equal(b1, b2)
    a3, _ = W.pertensor_pair(64, 48, 32, seed=4)
    assert not np.array_equal(a1, a3)
    assert a1.dtype == np.float32 and a1.shape == (64, 32) and b1.shape == (32, 48)


def test_llm_linear_outlier_channels():
    ch = W.outlier_channels(8192)
    assert ch.size == 82 and len(np.unique(ch)) == 82
    a, w = W.llm_linear(16, 64, 8192)
    amp = np.abs(a).mean(axis=0)
    assert set(np.argsort(amp)[-82:]) == set(ch)            # the x20 channels dominate
    assert abs(float(w.std()) - 0.02) < 0.002
    a_big, _ = W.llm_linear(128, 64, 8192)
    assert np.array_equal(W.outlier_channels(8192), ch)


def test_blockscaled_tile_factors_range():
    f = W.tile_factors(256, 512, 0, "A")
    assert f.shape == (8, 16) and f.min() >= 1e-2 and f.max() <= 1e2
    a, b = W.blockscaled_pair(64, 64, 64)
    assert a.shape == (64, 64) and np.isfinite(a).all()


def test_moe_counts_and_offsets():
    c = W.zipf_counts(8, 16384)
    assert c.sum() == 16384 and np.all(np.diff(c) < 0)     # Zipf: decreasing popularity
    off = W.offsets_from_counts(c)
    assert off[0] == 0 and off[-1] == 16384 and np.all(np.diff(off) >= 0)
    x, w, off2 = W.moe(E=3, T=50, K=32, N=16)
    assert x.shape == (50, 32) and w.shape == (3, 32, 16) and off2[-1] == 50
