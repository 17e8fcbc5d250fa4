"""GPU parity of the preshuffled scale layout (block 32): the scale bytes of 8 consecutive rows
for one block form one 8-byte word (the order the m = 1 GEMV reads them).  mx_quantize writes
the same codes and the same scale bytes as the oracle's row-major quantizer, at the positions
the layout defines, with zeros in the padding; mx_dequantize reads them back bit-exactly; the
m = 1 GEMV on preshuffled scales gives the row-major GEMV's outputs bit for bit and is within
2e-5 sum|x w| of the oracle."""
import numpy as np
import pytest
import torch

import microscaling_fp4_weight_amd as mx
import oracle
import synth
from gpu_util import (DEV, assert_gemm_close, bf16_dev, f32_dev, preshuffled_padding_positions,
                      preshuffled_positions, to_host_bits)

pytestmark = pytest.mark.gpu
FMTS = ["e4m3", "ue5m3", "e8m0"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mx.lib()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("rows,k", [(8, 2048), (13, 4224), (300, 8192), (5, 64), (17, 2112)])
@pytest.mark.parametrize("g", [1.0, 0.37])
def test_quantize_dequantize_preshuffled(dtype, fmt, rows, k, g):
    g = float(np.float32(g))
    x = synth.normal((rows, k), dtype, f"ps.{dtype}.{rows}.{k}", 0.02, 0.01, 20.0)
    xd = bf16_dev(x) if dtype == "bf16" else f32_dev(x)
    codes, scales = mx.mx_quantize(xd, 32, fmt, g, layout="preshuffled")
    assert scales.numel() == mx.mx_scale_bytes(rows, k, 32, "preshuffled")
    rc, rs = oracle.quantize(x, 32, fmt, g)
    got = to_host_bits(scales)
    np.testing.assert_array_equal(to_host_bits(codes), rc)
    np.testing.assert_array_equal(got[preshuffled_positions(rows, k)], rs)
    assert np.all(got[preshuffled_padding_positions(rows, k)] == 0)
    for out in ("f32", "bf16"):
        dt = torch.float32 if out == "f32" else torch.bfloat16
        y = mx.mx_dequantize(codes, scales, k, 32, fmt, g, out_dtype=dt, layout="preshuffled")
        ref = oracle.dequantize(rc, rs, k, 32, fmt, g, out)
        yb = to_host_bits(y)
        np.testing.assert_array_equal(yb.view(np.uint32) if out == "f32" else yb,
                                      ref.view(np.uint32) if out == "f32" else ref)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k", [(4096, 4096), (1000, 4224), (77, 2112), (8, 64)])
@pytest.mark.parametrize("g", [1.0, 0.37])
def test_gemv_preshuffled(fmt, n, k, g):
    g = float(np.float32(g))
    x = synth.normal((1, k), "bf16", f"psg.x.{k}", 1.0)
    w = synth.normal((n, k), "bf16", f"psg.w.{n}.{k}", 0.02, 0.01, 20.0)
    wd = bf16_dev(w)
    cp, sp = mx.mx_quantize(wd, 32, fmt, g, layout="preshuffled")
    cr, sr = mx.mx_quantize(wd, 32, fmt, g)
    xd = bf16_dev(x)
    for dt in (torch.float32, torch.bfloat16):
        yp = mx.mx_gemm(xd, cp, sp, 32, fmt, g, "a16", out_dtype=dt, layout="preshuffled")
        yr = mx.mx_gemm(xd, cr, sr, 32, fmt, g, "a16", out_dtype=dt)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_host_bits(yp), to_host_bits(yr))
    rc, rs = oracle.quantize(w, 32, fmt, g)
    yref, aref = oracle.gemm(x, rc, rs, 32, fmt, g)
    assert_gemm_close(to_host_bits(yp.float()), yref, aref, True, f"preshuffled gemv {fmt} {n}x{k}")


def test_preshuffled_gemm_needs_m1():
    x = bf16_dev(synth.normal((4, 256), "bf16", "psm.x", 1.0))
    w = bf16_dev(synth.normal((64, 256), "bf16", "psm.w", 0.02))
    c, s = mx.mx_quantize(w, 32, "e8m0", layout="preshuffled")
    with pytest.raises(mx.MXError):
        mx.mx_gemm(x, c, s, 32, "e8m0", 1.0, "a16", layout="preshuffled")
