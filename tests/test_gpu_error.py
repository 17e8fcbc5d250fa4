"""GPU parity of mx_quant_error (the device-side error split, hotelren.com/news/2192771
article "量化技术演进与微缩量化原理" section 2.2) against the CPU oracle's mse_split: the same
codes and scales are implied (both follow the quantizer bit for bit), so the per-element
errors are identical and only the order of the fp64 sums differs -- the means agree to a
relative 1e-12 and the block counts exactly."""
import numpy as np
import pytest
import torch

import microscaling_fp4_weight_amd as mx
import oracle
import synth
from gpu_util import DEV, bf16_dev, edge_tensor, f32_dev, to_host_bits

pytestmark = pytest.mark.gpu

KEYS = ("elem", "max", "zero", "total")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mx.lib()


def check(x_host, xd, block, fmt, g=1.0, x_hat=None):
    ref = oracle.mse_split(x_host, block, fmt, g)
    out = mx.mx_quant_error(xd, block, fmt, g, x_hat=x_hat).cpu().numpy()
    for i, key in enumerate(KEYS):
        assert out[i] == pytest.approx(ref[key], rel=1e-12, abs=1e-300), (key, block, fmt, g)
    assert int(out[4]) == ref["blocks"]
    assert int(out[5]) == ref["zero_blocks"]
    assert int(out[6]) == ref["max_not6"]
    return out


@pytest.mark.parametrize("fmt", ["e4m3", "ue5m3", "e8m0"])
@pytest.mark.parametrize("block", [4, 8, 16, 32, 64, 128, 256])
@pytest.mark.parametrize("sigma", [0.005, 0.1])
def test_error_split_bf16(fmt, block, sigma):
    x = synth.normal((96, 2048), "bf16", f"er.{sigma}", sigma, 0.001, 20.0)
    check(x, bf16_dev(x), block, fmt)


def test_error_split_tiny_round_trip_config():
    # fp32 256 x 256 ~ N(0, 0.02^2), 1% entries x20, block 32, E4M3
    w = synth.c1_weight()
    check(w, torch.from_numpy(w).to(DEV), 32, "e4m3")


@pytest.mark.parametrize("fmt", ["e4m3", "ue5m3", "e8m0"])
@pytest.mark.parametrize("block", [4, 32, 256])
def test_error_split_tensor_scale(fmt, block):
    x = synth.normal((64, 1024), "bf16", "er.g", 0.01, 0.01, 20.0)
    g = float(np.float32(0.0137))
    check(x, bf16_dev(x), block, fmt, g)
    xf = synth.bf16_to_f32(x)  # the same values as fp32 input
    check(xf, torch.from_numpy(xf).to(DEV), block, fmt, g)


def test_error_split_flushed_tensor():
    # sigma 1e-4 under E4M3: every block flushes (scale 0); the zero term carries everything
    x = synth.normal((32, 512), "bf16", "er.flush", 1e-4)
    out = check(x, bf16_dev(x), 32, "e4m3")
    assert out[5] == out[4] and out[0] == 0.0 and out[1] == 0.0


def test_error_split_strided_and_deterministic():
    x = synth.normal((40, 800), "bf16", "er.s", 0.02, 0.01, 20.0)
    xd = bf16_dev(x)[:, :736]
    ref_host = np.ascontiguousarray(x[:, :736])
    a = check(ref_host, xd, 32, "ue5m3")
    b = mx.mx_quant_error(xd, 32, "ue5m3").cpu().numpy()
    assert a.tobytes() == b.tobytes()


def test_error_split_llama7b_ffn_full():
    # the full sweep tensor at one configuration (sigma 0.02, block 32, E4M3)
    w = synth.c2_weight(0.02)
    check(w, bf16_dev(w), 32, "e4m3")


def dev(x):
    return bf16_dev(x) if x.dtype == np.uint16 else f32_dev(x)


def check_fake_quant(x, block, fmt, g, ld=None):
    """Error split plus x^ (the dequantized tensor) bit-exact against the oracle's quantize
    then dequantize; ld > k puts x and x^ in wider buffers (row stride ld)."""
    rows, k = x.shape
    if ld is None:
        xd = dev(x)
    else:
        wide = np.zeros((rows, ld), dtype=x.dtype)
        wide[:, :k] = x
        xd = dev(wide)[:, :k]
    xh_full = torch.full((rows, ld or k), -1.0, dtype=xd.dtype, device=DEV)
    xh = xh_full[:, :k]
    check(x, xd, block, fmt, g, x_hat=xh)
    codes, scales = oracle.quantize(x, block, fmt, g)
    ref = oracle.dequantize(codes, scales, k, block, fmt, g, "bf16" if x.dtype == np.uint16 else "f32")
    got = to_host_bits(xh.contiguous())
    if x.dtype == np.uint16:
        np.testing.assert_array_equal(got, ref)
    else:
        np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))
    if ld is not None:  # the padding columns are untouched
        assert torch.all(xh_full[:, k:] == -1.0)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fmt", ["e4m3", "ue5m3", "e8m0"])
@pytest.mark.parametrize("block", [4, 32, 256])
@pytest.mark.parametrize("g", [1.0, 0.0137])
def test_fake_quant_fast_path(dtype, fmt, block, g):
    g = float(np.float32(g))
    x = synth.normal((48, 1024), dtype, f"fq.{dtype}", 0.02, 0.01, 20.0)
    check_fake_quant(x, block, fmt, g)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fmt", ["e4m3", "e8m0"])
@pytest.mark.parametrize("block,k,ld", [(8, 504, None), (4, 36, None), (32, 512, 516), (64, 512, 514)])
@pytest.mark.parametrize("g", [1.0, 0.37])
def test_fake_quant_generic_path(dtype, fmt, block, k, ld, g):
    # k % 32 != 0 or a row stride that is not a multiple of 16 bytes: one thread per block
    g = float(np.float32(g))
    x = synth.normal((37, k), dtype, f"fqg.{dtype}.{k}", 0.05, 0.02, 20.0)
    check_fake_quant(x, block, fmt, g, ld)


@pytest.mark.parametrize("fmt", ["e4m3", "ue5m3", "e8m0"])
@pytest.mark.parametrize("block", [8, 32, 128])
@pytest.mark.parametrize("ld", [None, 516])
def test_error_split_edge_values(fmt, block, ld):
    # every scale byte, ties at the maximum with both signs, signed zeros, flush boundaries,
    # subnormals and near-overflow blocks; ld = 516 takes the generic path
    check_fake_quant(edge_tensor(512), block, fmt, 1.0, ld)


@pytest.mark.parametrize("block", [4, 64, 256])
def test_error_split_all_ties(block):
    # every element at +-amax: the whole block's error is one value; the max term takes one
    # element per block and the element term the rest
    rng = np.random.default_rng(7)
    mags = (rng.integers(1, 100, size=(16, 1)) * 0.0173).astype(np.float32)
    signs = np.where(rng.random((16, 512)) < 0.5, -1.0, 1.0).astype(np.float32)
    x = (mags * signs).astype(np.float32)
    for fmt in ("e4m3", "ue5m3", "e8m0"):
        check_fake_quant(x, block, fmt, 1.0)
        check_fake_quant(x, block, fmt, 1.0, ld=516)
