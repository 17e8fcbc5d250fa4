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
from gpu_util import DEV, bf16_dev

pytestmark = pytest.mark.gpu

KEYS = ("elem", "max", "zero", "total")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mx.lib()


def check(x_host, xd, block, fmt, g=1.0):
    ref = oracle.mse_split(x_host, block, fmt, g)
    out = mx.mx_quant_error(xd, block, fmt, g).cpu().numpy()
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
def test_error_split_tensor_scale(fmt):
    x = synth.normal((64, 1024), "bf16", "er.g", 0.01, 0.01, 20.0)
    check(x, bf16_dev(x), 32, fmt, float(np.float32(0.0137)))


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
