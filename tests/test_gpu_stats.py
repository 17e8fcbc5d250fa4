"""GPU parity of mx_tensor_stats (the statistic behind the block-size policy of
hotelren.com/news/2192771, article "量化技术演进与微缩量化原理", section 6 item 2) against the
oracle's two-pass fp64 tensor_stats: max |x| exact; mean and standard deviation to a relative
1e-12 (only the order of the fp64 sums differs; the mean also gets an absolute allowance of
1e-14 max|x| for near-zero means); the policy's block size equal."""
import numpy as np
import pytest
import torch

import microscaling_fp4_weight_amd as mx
import oracle
import synth
from gpu_util import DEV, bf16_dev, f32_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mx.lib()


def dev(x):
    return bf16_dev(x) if x.dtype == np.uint16 else f32_dev(x)


def check(x_host, xd):
    ref = oracle.tensor_stats(x_host)
    got = mx.mx_tensor_stats(xd).cpu().numpy()
    assert got[2] == ref["absmax"]
    assert got[0] == pytest.approx(ref["mean"], rel=1e-12, abs=1e-14 * ref["absmax"])
    if np.isnan(ref["std"]):
        assert np.isnan(got[1])
    else:
        assert got[1] == pytest.approx(ref["std"], rel=1e-12, abs=1e-300)
        assert mx.mx_adaptive_block_size(float(got[1])) == oracle.adaptive_block_size(ref["std"])
    return got


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(1, 8), (3, 40), (37, 1000), (256, 4096), (5, 8 * 40001)])
def test_stats_vector_path(dtype, shape):
    x = synth.normal(shape, dtype, f"st.{dtype}.{shape}", 0.03, 0.01, 20.0)
    check(x, dev(x))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape,ld", [((7, 13), None), ((33, 1002), None), ((20, 512), 515), ((9, 64), 66)])
def test_stats_element_path(dtype, shape, ld):
    # k % 8 != 0 or a row stride that is not a multiple of 16 bytes: one element per unit
    x = synth.normal(shape, dtype, f"ste.{dtype}.{shape}", 0.5)
    if ld is None:
        check(x, dev(x))
    else:
        wide = np.zeros((shape[0], ld), dtype=x.dtype)
        wide[:, :shape[1]] = x
        check(x, dev(wide)[:, :shape[1]])


def test_stats_closed_forms():
    x = np.arange(1, 4097, dtype=np.float32).reshape(16, 256)
    got = check(x, f32_dev(x))
    assert got[0] == 2048.5 and got[2] == 4096.0
    c = np.full((64, 128), -0.375, dtype=np.float32)
    got = check(c, f32_dev(c))
    assert got[0] == -0.375 and got[1] == 0.0
    one = np.array([[3.0]], dtype=np.float32)
    got = check(one, f32_dev(one))
    assert np.isnan(got[1]) and got[0] == 3.0


def test_stats_llama7b_ffn_and_policy():
    for sigma, block in ((0.005, 128), (0.02, 64), (0.1, 32)):
        w = synth.c2_weight(sigma)
        wd = bf16_dev(w)
        got = check(w, wd)
        assert mx.mx_adaptive_block_size(float(got[1])) == block
        again = mx.mx_tensor_stats(wd).cpu().numpy()
        assert again.tobytes() == got.tobytes()  # fixed summation order
