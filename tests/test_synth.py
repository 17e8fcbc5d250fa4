"""The seeded input generator: determinism, slice independence, dtype rounding, statistics."""
import numpy as np
import torch


def test_deterministic_and_sliceable(syn):
    a = syn.normal((64, 96), "bf16", "t.det", 0.02, 0.01, 20.0)
    b = syn.normal((64, 96), "bf16", "t.det", 0.02, 0.01, 20.0)
    np.testing.assert_array_equal(a, b)
    part = syn.normal((64, 96), "bf16", "t.det", 0.02, 0.01, 20.0, row0=17, nrows=9)
    np.testing.assert_array_equal(part, a[17:26])
    c = syn.normal((64, 96), "bf16", "t.other", 0.02, 0.01, 20.0)
    assert not np.array_equal(a, c)


def test_bf16_is_rne_of_f32(syn):
    f = syn.normal((128, 256), "f32", "t.rne", 0.7, 0.01, 20.0)
    b = syn.normal((128, 256), "bf16", "t.rne", 0.7, 0.01, 20.0)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(b, ref)


def test_statistics(syn):
    x = syn.normal((512, 4096), "f32", "t.stats", 0.02).astype(np.float64)
    assert abs(x.mean()) < 1e-4 and abs(x.std() - 0.02) < 2e-4
    y = syn.normal((512, 4096), "f32", "t.stats", 0.02, 0.01, 20.0).astype(np.float64)
    frac = np.mean(np.abs(y - x) > 0)
    assert 0.0095 < frac < 0.0105
    np.testing.assert_allclose(y[y != x], 20 * x[y != x], rtol=1e-6)


def test_banded(syn):
    w = syn.banded_bf16((64, 512), "t.band", 16, 4, 3, 0.01, 0.02)
    wf = syn.bf16_to_f32(w).astype(np.float64).reshape(16, 4, 512)
    sd = wf.std(axis=(1, 2))
    for b in range(16):
        assert abs(sd[b] - (0.02 if b % 4 == 3 else 0.01)) < 0.0015 * (2 if b % 4 == 3 else 1)
    part = syn.banded_bf16((64, 512), "t.band", 16, 4, 3, 0.01, 0.02, row0=12, nrows=8)
    np.testing.assert_array_equal(part, w[12:20])
