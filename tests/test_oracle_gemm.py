"""Oracle pins: the fp64 matmul Y = Xhat . What^T (gtnt.cn/news/16247, "为什么我们需要4-bit浮点
量化", section 3.1: dequantize, then matmul).

 * against numpy's float64 matmul of the oracle-dequantized weight (a library routine) on
   non-square shapes, so a transposed operand or a wrong block index fails;
 * against exact rational sums on small k;
 * W4A4: the activations are MX-quantized (block 32, E8M0, per-tensor 1) and dequantized first;
 * the sampled (row, column) form equals the full product.
"""
from fractions import Fraction

import numpy as np
import pytest


def _xw(syn, m, n, k, seed_name, sigma_w=0.02):
    x = syn.normal((m, k), "bf16", f"{seed_name}.x", 1.0)
    w = syn.normal((n, k), "bf16", f"{seed_name}.w", sigma_w, 0.01, 20.0)
    return x, w


@pytest.mark.parametrize("fmt,block,g", [("e8m0", 32, 1.0), ("e4m3", 16, 1.0),
                                         ("ue5m3", 64, float(np.float32(0.37))), ("e8m0", 4, 2.0)])
def test_gemm_vs_numpy(ox, syn, fmt, block, g):
    m, n, k = 5, 37, 384
    x, w = _xw(syn, m, n, k, f"gemm.{fmt}.{block}")
    c, s = ox.quantize(w, block, fmt, g)
    y, a = ox.gemm(x, c, s, block, fmt, g)
    assert y.shape == (m, n)
    # What as exact doubles: e*s*g (dequantize to fp32 with g = 1 is exact, then times g)
    wh = ox.dequantize(c, s, k, block, fmt, 1.0, "f32").astype(np.float64) * g
    xh = syn.bf16_to_f32(x).astype(np.float64)
    ref = xh @ wh.T
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12 * np.max(a))
    np.testing.assert_allclose(a, np.abs(xh) @ np.abs(wh).T, rtol=1e-13)


def test_gemm_exact_small_k(ox, syn):
    m, n, k = 2, 3, 64
    x, w = _xw(syn, m, n, k, "gemm.exact")
    c, s = ox.quantize(w, 32, "ue5m3")
    y, _ = ox.gemm(x, c, s, 32, "ue5m3")
    wh = ox.dequantize(c, s, k, 32, "ue5m3", 1.0, "f32")
    xh = syn.bf16_to_f32(x)
    for i in range(m):
        for j in range(n):
            exact = sum(Fraction(float(xh[i, kk])) * Fraction(float(wh[j, kk])) for kk in range(k))
            assert abs(Fraction(y[i, j]) - exact) <= abs(exact) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)


def test_gemm_w4a4(ox, syn):
    m, n, k = 4, 19, 256
    x, w = _xw(syn, m, n, k, "gemm.a4")
    c, s = ox.quantize(w, 32, "e8m0")
    y, a = ox.gemm(x, c, s, 32, "e8m0", 1.0, mode="a4")
    xc, xs = ox.quantize(x, 32, "e8m0")
    xh = ox.dequantize(xc, xs, k, 32, "e8m0", 1.0, "f32").astype(np.float64)
    wh = ox.dequantize(c, s, k, 32, "e8m0", 1.0, "f32").astype(np.float64)
    np.testing.assert_allclose(y, xh @ wh.T, rtol=0, atol=1e-12 * np.max(a))
    # and it differs from W4A16 (the activations really were quantized)
    y16, _ = ox.gemm(x, c, s, 32, "e8m0", 1.0, mode="a16")
    assert np.max(np.abs(y - y16)) > 1e-3 * np.max(np.abs(y16))


def test_gemm_sampled_equals_full(ox, syn):
    m, n, k = 6, 40, 128
    x, w = _xw(syn, m, n, k, "gemm.sample")
    c, s = ox.quantize(w, 32, "e4m3")
    yf, af = ox.gemm(x, c, s, 32, "e4m3")
    rows, cols = [5, 0, 3], [39, 2, 17, 0]
    ys, as_ = ox.gemm(x, c, s, 32, "e4m3", mrows=rows, ncols=cols)
    np.testing.assert_array_equal(ys, yf[np.ix_(rows, cols)])
    np.testing.assert_array_equal(as_, af[np.ix_(rows, cols)])


def test_gemm_rejects_bad_args(ox, syn):
    x, w = _xw(syn, 2, 3, 64, "gemm.bad")
    c, s = ox.quantize(w, 32, "e8m0")
    with pytest.raises(ValueError):
        ox.gemm(x, c, s, 32, "e8m0", mrows=[2])
    with pytest.raises(ValueError):
        ox.quantize(w[:, :48], 32, "e8m0")  # k not a multiple of the block
