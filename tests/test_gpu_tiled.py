"""GPU parity of the tiled scale layout (include/mx.h, MX_LAYOUT_TILED): the scale bytes
are the oracle's row-major scales placed at the positions the layout defines (padding
blocks of a row's last 256-element stage read 0), the codes are those of the row-major
layout, dequantization is bit-identical, and the W4A4 product with tiled weight scales
equals the one with row-major weight scales bit for bit and the oracle within the matmul
tolerance.  The position formula is written out here from the header's definition, apart
from the library."""
import numpy as np
import pytest
import torch

import microscaling_fp4_weight_amd as mx
import oracle
import synth
from gpu_util import DEV, assert_gemm_close, bf16_dev, padding_positions, tiled_positions, to_host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mx.lib()


@pytest.mark.parametrize("rows,k", [(300, 8192), (256, 4224), (7, 96), (513, 1024)])
@pytest.mark.parametrize("fmt", ["e8m0", "e4m3"])
@pytest.mark.parametrize("g", [1.0, 0.37])
def test_quantize_tiled(rows, k, fmt, g):
    g = float(np.float32(g))
    x = synth.normal((rows, k), "bf16", f"tl.{rows}.{k}", 0.5, 0.01, 30.0)
    c_ref, s_ref = oracle.quantize(x, 32, fmt, g)
    xd = bf16_dev(x)
    nbytes = mx.mx_scale_bytes(rows, k, 32, "tiled")
    assert nbytes == -(-rows // 256) * -(-k // 256) * 2048
    scales = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=DEV)  # poison the padding
    codes, scales = mx.mx_quantize(xd, 32, fmt, g, layout="tiled", scales=scales)
    torch.cuda.synchronize()
    got = to_host_bits(scales)
    np.testing.assert_array_equal(to_host_bits(codes), c_ref)
    np.testing.assert_array_equal(got[tiled_positions(rows, k)], s_ref)
    pad = padding_positions(rows, k)
    assert np.all(got[pad] == 0), "padding blocks of the last stage must read 0"
    # dequantization from tiled scales is the row-major result bit for bit
    for dt in (torch.float32, torch.bfloat16):
        y_t = mx.mx_dequantize(codes, scales, k, 32, fmt, g, out_dtype=dt, layout="tiled")
        y_r = mx.mx_dequantize(codes, torch.from_numpy(s_ref).to(DEV), k, 32, fmt, g, out_dtype=dt)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_host_bits(y_t), to_host_bits(y_r))


def test_quantize_tiled_f32_generic_rows():
    # fp32 input with a row stride that is not a multiple of 16 bytes: the one-block-per-thread
    # kernel writes the tiled positions too
    rows, k = 40, 288
    x = synth.normal((rows, k + 1), "f32", "tl.gen", 1.0)
    c_ref, s_ref = oracle.quantize(np.ascontiguousarray(x[:, :k]), 32, "e8m0", 1.0)
    xd = torch.from_numpy(x).to(DEV)[:, :k]
    nbytes = mx.mx_scale_bytes(rows, k, 32, "tiled")
    scales = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=DEV)
    codes, scales = mx.mx_quantize(xd, 32, "e8m0", layout="tiled", scales=scales)
    torch.cuda.synchronize()
    got = to_host_bits(scales)
    np.testing.assert_array_equal(to_host_bits(codes), c_ref)
    np.testing.assert_array_equal(got[tiled_positions(rows, k)], s_ref)
    assert np.all(got[padding_positions(rows, k)] == 0)


@pytest.mark.parametrize("mnk", [(200, 300, 640), (256, 512, 4224), (33, 1000, 2048)])
def test_gemm_a4_tiled_weights(mnk):
    m, n, k = mnk
    x = synth.normal((m, k), "bf16", f"tg.x.{m}", 1.0)
    w = synth.normal((n, k), "bf16", f"tg.w.{n}", 0.02, 0.01, 20.0)
    c, s = oracle.quantize(w, 32, "e8m0", 1.0)
    xd, wd = bf16_dev(x), bf16_dev(w)
    ct, st = mx.mx_quantize(wd, 32, "e8m0", layout="tiled")
    cd, sd = torch.from_numpy(c).to(DEV), torch.from_numpy(s).to(DEV)
    for dt in (torch.float32, torch.bfloat16):
        y_t = mx.mx_gemm(xd, ct, st, 32, "e8m0", 1.0, "a4", out_dtype=dt, layout="tiled")
        y_r = mx.mx_gemm(xd, cd, sd, 32, "e8m0", 1.0, "a4", out_dtype=dt)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_host_bits(y_t), to_host_bits(y_r))
    yref, aref = oracle.gemm(x, c, s, 32, "e8m0", 1.0, "a4")
    assert_gemm_close(to_host_bits(y_t.float()), yref, aref, True, f"a4 tiled {mnk}")


def test_gemm_tiled_rejected_where_unsupported():
    m, n, k = 4, 64, 256
    xd = bf16_dev(synth.normal((m, k), "bf16", "tr.x", 1.0))
    ct, st = mx.mx_quantize(bf16_dev(synth.normal((n, k), "bf16", "tr.w", 0.02)), 32, "e8m0",
                            layout="tiled")
    with pytest.raises(mx.MXError) as e:
        mx.mx_gemm(xd, ct, st, 32, "e8m0", 1.0, "a16", layout="tiled")
    assert e.value.status == -2


@pytest.mark.parametrize("layout", ["rowmajor", "tiled"])
@pytest.mark.parametrize("mnk", [(256, 66560, 256), (512, 16640, 256), (300, 33000, 128)])
def test_gemm_a4_full_and_half_tiles(layout, mnk):
    """Shapes whose 256 x 256 tile count leaves a partial last round over the 256 CUs: 260
    tiles (256 full + 4 run as 8 half tiles), 130 tiles (all full: the round is more than half
    used), 258 tiles with a ragged last n-tile (2 run as half tiles).  Weights quantized on
    the GPU, their sampled rows checked against the oracle; outputs sampled in every kind of
    tile, including the half tiles at the end of n."""
    m, n, k = mnk
    x = synth.normal((m, k), "bf16", f"fh.x.{m}", 1.0)
    w = synth.normal((n, k), "bf16", f"fh.w.{n}", 0.02, 0.01, 20.0)
    wd = bf16_dev(w)
    cd, sd = mx.mx_quantize(wd, 32, "e8m0", layout=layout)
    del wd
    cols = np.array([0, 5, 1000, n // 2, n - 300, n - 129, n - 128, n - 1])
    rows = np.array([0, 1, m // 2, m - 1])
    rc, rs = oracle.quantize(w[cols], 32, "e8m0", 1.0)
    np.testing.assert_array_equal(to_host_bits(cd[cols]), rc)
    xd = bf16_dev(x)
    yref, aref = oracle.gemm(x[rows], rc, rs, 32, "e8m0", 1.0, "a4")
    for dt in (torch.float32, torch.bfloat16):
        y = mx.mx_gemm(xd, cd, sd, 32, "e8m0", 1.0, "a4", out_dtype=dt, layout=layout)
        torch.cuda.synchronize()
        got = to_host_bits(y.float())[rows][:, cols]
        assert_gemm_close(got, yref, aref, dt == torch.bfloat16, f"a4 {layout} {mnk} {dt}")
