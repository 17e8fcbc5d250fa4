"""Oracle pins: the block-size policy of hotelren.com/news/2192771 (article
"量化技术演进与微缩量化原理"): section 6 item 2 (block size from the tensor's standard
deviation: below 0.01 -> 128, below 0.1 -> 64, else 32) and section 5.1 item 1 (Q/K/V 64,
FFN gate/up 32, output 128), and the statistics the first one reads.

 * thresholds at, just below and just above each boundary value the page prints;
 * tensor_stats against closed forms (1..n, a constant tensor, two values) and against
   numpy's own std(ddof=1) on random data, and its bf16 reading against explicit widening;
 * the policy applied to the workload's three standard deviations picks three different
   block sizes.
"""
import numpy as np
import pytest


@pytest.mark.parametrize("sigma,block", [
    (0.0, 128), (0.005, 128), (np.nextafter(0.01, 0.0), 128), (0.01, 64), (0.02, 64),
    (0.05, 64), (np.nextafter(0.1, 0.0), 64), (0.1, 32), (0.5, 32), (3.0, 32),
    (float("nan"), 32),  # NaN passes neither test: the last branch
])
def test_adaptive_block_size(ox, sigma, block):
    assert ox.adaptive_block_size(sigma) == block


def test_layer_block_size(ox):
    assert ox.layer_block_size("qkv") == 64
    assert ox.layer_block_size("ffn_gate_up") == 32
    assert ox.layer_block_size("output") == 128
    with pytest.raises(KeyError):
        ox.layer_block_size("embedding")


def test_stats_closed_forms(ox):
    n = 1000
    x = np.arange(1, n + 1, dtype=np.float32).reshape(10, 100)
    r = ox.tensor_stats(x)
    assert r["mean"] == (n + 1) / 2
    assert r["std"] == pytest.approx(np.sqrt(n * (n + 1) / 12), rel=1e-15)  # var of 1..n, n-1 form
    assert r["absmax"] == n
    c = np.full((3, 64), -0.375, dtype=np.float32)
    r = ox.tensor_stats(c)
    assert r["mean"] == -0.375 and r["std"] == 0.0 and r["absmax"] == 0.375
    two = np.array([[-1.5, 2.5]], dtype=np.float32)
    r = ox.tensor_stats(two)
    assert r["mean"] == 0.5 and r["std"] == pytest.approx(np.sqrt(8.0), rel=1e-15)
    assert np.isnan(ox.tensor_stats(np.array([[4.0]], dtype=np.float32))["std"])


def test_stats_against_numpy(ox, syn):
    x = syn.normal((64, 1024), "f32", "stats.np", 0.02, 0.01, 20.0)
    r = ox.tensor_stats(x)
    v = x.astype(np.float64)
    assert r["mean"] == pytest.approx(v.mean(), rel=1e-12, abs=1e-18)
    assert r["std"] == pytest.approx(v.std(ddof=1), rel=1e-12)
    assert r["absmax"] == np.abs(v).max()
    b = syn.normal((64, 1024), "bf16", "stats.bf", 0.07)
    rb = ox.tensor_stats(b)
    wide = syn.bf16_to_f32(b).astype(np.float64)
    assert rb["std"] == pytest.approx(wide.std(ddof=1), rel=1e-12)
    assert rb["absmax"] == np.abs(wide).max()


def test_policy_on_the_sweep_sigmas(ox, syn):
    # rows of the three sweep tensors (sigma 0.005, 0.02, 0.1 with 0.1% outliers x20): the
    # measured std lands in three different policy bands
    picks = []
    for sigma in (0.005, 0.02, 0.1):
        w = syn.c2_weight(sigma, row0=0, nrows=256)
        s = ox.tensor_stats(w)["std"]
        assert s == pytest.approx(sigma * np.sqrt(1 + 0.001 * 399), rel=0.03)  # outliers widen it
        picks.append(ox.adaptive_block_size(s))
    assert picks == [128, 64, 32]
