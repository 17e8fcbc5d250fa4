"""GPU parity of the FP8 weight fallback (hotelren.com/news/2192771, article
"量化技术演进与微缩量化原理", section 5.3 item 1 and section 6 item 1) through the C ABI against
the oracle: E4M3 codes and scale bytes bit-exact, dequantized values bit-exact, the W8A16
product within |dY| <= 2e-5 * sum|x w| (plus half a bf16 ulp of Y for bf16 output)."""
import numpy as np
import pytest
import torch

import microscaling_fp4_weight_amd as mx
import oracle
import synth
from gpu_util import DEV, assert_gemm_close, bf16_dev, edge_tensor, f32_dev, to_host_bits

pytestmark = pytest.mark.gpu
FMTS = ["e4m3", "ue5m3", "e8m0"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mx.lib()


def dev(x):
    return bf16_dev(x) if x.dtype == np.uint16 else f32_dev(x)


def check_quant(x, block, fmt, g=1.0, ld=None):
    rows, k = x.shape
    if ld is None:
        xd = dev(x)
    else:
        wide = np.zeros((rows, ld), dtype=x.dtype)
        wide[:, :k] = x
        xd = dev(wide)[:, :k]
    c, s = mx.mx_quantize_fp8(xd, block, fmt, g)
    rc, rs = oracle.quantize_fp8(x, block, fmt, g)
    np.testing.assert_array_equal(to_host_bits(s), rs)
    np.testing.assert_array_equal(to_host_bits(c), rc)
    return c, s, rc, rs


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("block", [4, 8, 16, 32, 64, 128, 256])
def test_quantize_fp8(dtype, fmt, block):
    x = synth.normal((24, 1024), dtype, f"q8.{dtype}", 0.3, 0.01, 20.0)
    check_quant(x, block, fmt)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("g", [0.37, 3.1e-3])
def test_quantize_fp8_tensor_scale(fmt, g):
    g = float(np.float32(g))
    x = synth.normal((16, 512), "bf16", "q8.g", 0.05, 0.01, 20.0)
    check_quant(x, 32, fmt, g)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("block", [8, 32, 128])
def test_quantize_fp8_edge_values(fmt, block):
    # every scale byte, every bf16 magnitude under a fixed maximum, ties, zeros, subnormals
    check_quant(edge_tensor(512), block, fmt)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape,block,ld", [((9, 36), 4, None), ((7, 100), 4, None), ((20, 512), 32, 516),
                                            ((3, 96), 32, None)])
def test_quantize_fp8_generic_path(dtype, shape, block, ld):
    # k % 8 != 0 or rows not 16-byte aligned: one thread per block
    x = synth.normal(shape, dtype, f"q8g.{dtype}.{shape}", 0.1, 0.02, 20.0)
    check_quant(x, block, "ue5m3", 1.0, ld)


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("block", [4, 32, 256])
@pytest.mark.parametrize("g", [1.0, 0.37])
def test_dequantize_fp8(out, fmt, block, g):
    g = float(np.float32(g))
    x = np.concatenate([synth.normal((12, 512), "bf16", "d8", 0.02, 0.01, 20.0), edge_tensor(512)[:40]])
    rc, rs = oracle.quantize_fp8(x, block, fmt, g)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    y = mx.mx_dequantize_fp8(torch.from_numpy(rc).to(DEV), torch.from_numpy(rs).to(DEV), block, fmt, g, out_dtype=dt)
    ref = oracle.dequantize_fp8(rc, rs, block, fmt, g, out)
    got = to_host_bits(y)
    if out == "f32":
        np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))
    else:
        np.testing.assert_array_equal(got, ref)


def test_dequantize_fp8_every_code_and_scale():
    # all 256 element bytes (0x7F / 0xFF read as NaN) under every finite scale byte of each format
    codes = np.tile(np.arange(256, dtype=np.uint8), (256, 1))
    for fmt in FMTS:
        scales = np.arange(256, dtype=np.uint8).reshape(256, 1).repeat(8, axis=1)
        ok = np.array([np.isfinite(oracle.scale_value(b, fmt)) for b in range(256)])
        c, s = codes[ok], scales[ok]
        for out in ("f32", "bf16"):
            dt = torch.float32 if out == "f32" else torch.bfloat16
            y = mx.mx_dequantize_fp8(torch.from_numpy(np.ascontiguousarray(c)).to(DEV),
                                     torch.from_numpy(np.ascontiguousarray(s)).to(DEV), 32, fmt, 1.0, out_dtype=dt)
            ref = oracle.dequantize_fp8(c, s, 32, fmt, 1.0, out)
            got = to_host_bits(y)
            if out == "f32":
                np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))
            else:
                np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("m", [1, 4, 16, 17, 100])
@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_fp8(m, fmt):
    k, n = 1024, 200
    x = synth.normal((m, k), "bf16", f"g8.x.{m}", 1.0)
    w = synth.normal((n, k), "bf16", "g8.w", 0.02, 0.01, 20.0)
    rc, rs = oracle.quantize_fp8(w, 32, fmt)
    cd, sd = torch.from_numpy(rc).to(DEV), torch.from_numpy(rs).to(DEV)
    yref, aref = oracle.gemm_fp8(x, rc, rs, 32, fmt)
    for dt in (torch.float32, torch.bfloat16):
        y = mx.mx_gemm_fp8(bf16_dev(x), cd, sd, 32, fmt, out_dtype=dt)
        torch.cuda.synchronize()
        assert_gemm_close(to_host_bits(y.float()), yref, aref, dt == torch.bfloat16, f"w8 m={m} {fmt} {dt}")


# The decode kernel with 2 or 4 groups of 16 weight rows per workgroup (taken for m <= 16 once n
# keeps at least 224 workgroups): n 7200 (2 groups, 225 workgroups), n 14337 (4 groups, the last
# workgroup holding a single row); a partial last 128-k window, m 3 and 16, g != 1.  Every output.
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m,n,k,g", [(3, 7200, 1280, 1.0), (16, 7200, 4096, 0.37), (16, 14337, 1280, 1.0),
                                     (5, 14337, 1280, 0.37)])
def test_gemm_fp8_row_groups(m, n, k, g, fmt):
    g = float(np.float32(g))
    x = synth.normal((m, k), "bf16", f"g8g.x.{m}", 1.0)
    w = synth.normal((n, k), "bf16", f"g8g.w.{n}.{k}", 0.02 / g, 0.01, 20.0)
    rc, rs = oracle.quantize_fp8(w, 32, fmt, g)
    cd, sd = torch.from_numpy(rc).to(DEV), torch.from_numpy(rs).to(DEV)
    yref, aref = oracle.gemm_fp8(x, rc, rs, 32, fmt, g)
    for dt in (torch.float32, torch.bfloat16):
        y = mx.mx_gemm_fp8(bf16_dev(x), cd, sd, 32, fmt, g, out_dtype=dt)
        torch.cuda.synchronize()
        assert_gemm_close(to_host_bits(y.float()), yref, aref, dt == torch.bfloat16, f"w8 groups {m}x{n}x{k} {fmt} {dt}")


@pytest.mark.parametrize("block", [4, 8, 16, 64, 128, 256])
def test_gemm_fp8_blocks_tail_and_scale(block):
    # k = 1280 (a partial last 128-k window), ragged n, per-tensor g
    m, n, k = 7, 77, 1280
    g = float(np.float32(0.0291))
    x = synth.normal((m, k), "bf16", "g8b.x", 1.0)
    w = synth.normal((n, k), "bf16", f"g8b.w.{block}", 0.5, 0.01, 20.0)
    rc, rs = oracle.quantize_fp8(w, block, "ue5m3", g)
    y = mx.mx_gemm_fp8(bf16_dev(x), torch.from_numpy(rc).to(DEV), torch.from_numpy(rs).to(DEV), block, "ue5m3", g,
                       out_dtype=torch.float32)
    torch.cuda.synchronize()
    yref, aref = oracle.gemm_fp8(x, rc, rs, block, "ue5m3", g)
    assert_gemm_close(to_host_bits(y), yref, aref, False, f"w8 block {block}")


def _gemm_fp8_case(m, n, k, fmt, g, tag, ldx=None, ldy=None):
    x = synth.normal((m, k), "bf16", f"g8t.x.{tag}", 1.0)
    w = synth.normal((n, k), "bf16", f"g8t.w.{tag}", 0.02 / g, 0.01, 20.0)
    rc, rs = oracle.quantize_fp8(w, 32, fmt, g)
    cd, sd = torch.from_numpy(rc).to(DEV), torch.from_numpy(rs).to(DEV)
    xd = bf16_dev(x)
    if ldx is not None:
        wide = torch.zeros((m, ldx), dtype=torch.bfloat16, device=DEV)
        wide[:, :k] = xd
        xd = wide[:, :k]
    yref, aref = oracle.gemm_fp8(x, rc, rs, 32, fmt, g)
    for dt in (torch.float32, torch.bfloat16):
        y = None
        if ldy is not None:
            y = torch.full((m, ldy), float("nan"), dtype=dt, device=DEV)[:, :n]
        y = mx.mx_gemm_fp8(xd, cd, sd, 32, fmt, g, out_dtype=dt, y=y)
        torch.cuda.synchronize()
        assert_gemm_close(to_host_bits(y.float()), yref, aref, dt == torch.bfloat16, f"w8 {tag} {fmt} {dt}")
        if ldy is not None:  # nothing written beyond the n columns of each row
            assert torch.isnan(y.as_strided((m, ldy - n), (ldy, 1), n)).all()


# Larger products run on the pipelined matrix-core kernels (scale windows of 512 k): for m > 128
# the wide one (256 x 256 tiles, k in stages of 64), else the one with 128 x 256 tiles and
# 128-k stages (the last shape); the library picks them when the estimated time is below the
# 16-row kernel's, which these shapes pass by a factor of 1.1 or more with every scale format.
# Every output is compared: several tiles with ragged tails in m and n (down to a single row
# and column), n-tile counts that are and are not multiples of 8 (two mappings of tiles to XCDs).
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("mnk", [(300, 6000, 1536), (129, 7937, 512), (200, 5000, 512), (128, 8000, 1536)])
def test_gemm_fp8_tiled(mnk, fmt):
    m, n, k = mnk
    _gemm_fp8_case(m, n, k, fmt, 1.0, f"{m}.{n}.{k}")


@pytest.mark.parametrize("fmt,ldy", [("ue5m3", 4003), ("e8m0", 4008)])
def test_gemm_fp8_tiled_tensor_scale_and_strides(fmt, ldy):
    # padded activation rows (ldx = k + 8); output rows of n + 3 (odd: chunk stores are off,
    # element stores on) or n + 8 (chunk stores on); per-tensor g
    g = float(np.float32(0.0291))
    _gemm_fp8_case(300, 4000, 1024, fmt, g, f"ld{ldy}", ldx=1032, ldy=ldy)


# m <= 2, block 32, k in {4096, 8192, 16384}, short streams: the sweeping GEMV with FP8 codes
# (2 KB chunks of 2048 k read as two 1 KB halves; a lane's 32 k span two blocks): one and
# several steps, uneven step counts, 1 / 2 / 4 rows per unit, one and two rows of X.
@pytest.mark.parametrize("m", [1, 2])
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k", [(1000, 4096), (8000, 4096), (2050, 8192), (777, 16384)])
def test_gemv_fp8_sweep(n, k, fmt, m):
    g = float(np.float32(0.37)) if fmt == "ue5m3" else 1.0
    x = synth.normal((m, k), "bf16", f"sw8.x.{k}.{m}", 1.0)
    w = synth.normal((n, k), "bf16", f"sw8.w.{n}.{k}", 0.02 / g, 0.01, 20.0)
    rc, rs = oracle.quantize_fp8(w, 32, fmt, g)
    cd, sd = torch.from_numpy(rc).to(DEV), torch.from_numpy(rs).to(DEV)
    yref, aref = oracle.gemm_fp8(x, rc, rs, 32, fmt, g)
    for dt in (torch.float32, torch.bfloat16):
        y = mx.mx_gemm_fp8(bf16_dev(x), cd, sd, 32, fmt, g, out_dtype=dt)
        torch.cuda.synchronize()
        assert_gemm_close(to_host_bits(y.float()), yref, aref, dt == torch.bfloat16, f"w8 sweep m={m} {fmt} {n}x{k} {dt}")


# Zero-scale blocks through the sweeping FP8-weight GEMV (with E4M3 / UE5M3 scales the mantissa
# of each lane's 16 elements, which lie in one 32-element block, multiplies their sum, so a
# zero scale must give a zero contribution):
# all-zero blocks and blocks below the FP8 flush threshold (a <= 448 s_min / 2 g-scaled:
# E4M3 0.44 g, UE5M3 1.7e-3 g), one and two rows of X.
@pytest.mark.parametrize("fmt,g", [("e8m0", 1.0), ("e4m3", 1.0), ("ue5m3", 0.37)])
@pytest.mark.parametrize("m", [1, 2])
def test_gemv_fp8_zero_and_flushed_blocks(fmt, g, m):
    g = float(np.float32(g))
    n, k = 96, 4096
    x = synth.normal((m, k), "bf16", f"gz8.x.{m}", 1.0)
    w32 = synth.normal((n, k), "f32", "gz8.w", 1.0)        # blocks well above every threshold
    blocks = w32.reshape(n, k // 32, 32)                  # the scale blocks
    blocks[::3, ::5] = 0.0
    tiny = {"e8m0": 0.0, "e4m3": 0.2, "ue5m3": 5e-4}[fmt]
    blocks[1::3, 1::4] *= tiny / 4
    w = torch.from_numpy(blocks.reshape(n, k)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    rc, rs = oracle.quantize_fp8(w, 32, fmt, g)
    assert (rs == 0).any()
    cd, sd = torch.from_numpy(rc).to(DEV), torch.from_numpy(rs).to(DEV)
    yref, aref = oracle.gemm_fp8(x, rc, rs, 32, fmt, g)
    for dt in (torch.float32, torch.bfloat16):
        y = mx.mx_gemm_fp8(bf16_dev(x), cd, sd, 32, fmt, g, out_dtype=dt)
        torch.cuda.synchronize()
        assert_gemm_close(to_host_bits(y.float()), yref, aref, dt == torch.bfloat16, f"w8 zero blocks {fmt} m={m} {dt}")


@pytest.mark.parametrize("fmt,g", [("e8m0", 1.0), ("e4m3", 1.0), ("ue5m3", 0.37)])
def test_fp8_full_tensor_exact(fmt, g):
    """FP8 fallback on the whole Llama-7B FFN weight (4096 x 11008 bf16, block 32): every code,
    scale byte and dequantized bf16 element equal to the oracle's (g = 1 takes the 32-element
    lane kernel, g != 1 the 8-element one)."""
    g = float(np.float32(g))
    w = synth.c2_weight(0.02)
    wd = bf16_dev(w)
    cd, sd = mx.mx_quantize_fp8(wd, 32, fmt, g)
    y = mx.mx_dequantize_fp8(cd, sd, 32, fmt, g, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    del wd
    rc, rs = oracle.quantize_fp8(w, 32, fmt, g)
    np.testing.assert_array_equal(to_host_bits(sd), rs, err_msg=f"scales {fmt}")
    np.testing.assert_array_equal(to_host_bits(cd), rc, err_msg=f"codes {fmt}")
    np.testing.assert_array_equal(to_host_bits(y), oracle.dequantize_fp8(rc, rs, 32, fmt, g, "bf16"),
                                  err_msg=f"dequantized {fmt}")


@pytest.mark.parametrize("fmt,g", [("e8m0", 1.0), ("ue5m3", 0.37)])
def test_gemm_fp8_wide_tiles_sampled(fmt, g):
    """W8A16 through the wide-tile kernel (m 1000 and n 28600, both ragged): sampled rows and
    columns against the oracle, fp32 and bf16 out."""
    g = float(np.float32(g))
    m, n, k = 1000, 28600, 1024
    x = synth.normal((m, k), "bf16", "gw8.x", 1.0)
    w = synth.normal((n, k), "bf16", "gw8.w", 0.02 / g, 0.01, 20.0)
    wd = bf16_dev(w)
    cd, sd = mx.mx_quantize_fp8(wd, 32, fmt, g)
    del wd
    cols = np.array([0, 1, 255, 256, 9999, 28415, 28416, 28599])
    rows = np.array([0, 1, 127, 128, 255, 256, 767, 768, 999])
    rc, rs = oracle.quantize_fp8(w[cols], 32, fmt, g)
    np.testing.assert_array_equal(to_host_bits(cd[cols]), rc)
    np.testing.assert_array_equal(to_host_bits(sd[cols]), rs)
    yref, aref = oracle.gemm_fp8(x[rows], rc, rs, 32, fmt, g)
    for dt in (torch.float32, torch.bfloat16):
        y = mx.mx_gemm_fp8(bf16_dev(x), cd, sd, 32, fmt, g, out_dtype=dt)
        torch.cuda.synchronize()
        assert_gemm_close(to_host_bits(y[rows][:, cols].float()), yref, aref, dt == torch.bfloat16,
                          f"w8 wide tiles {fmt} {dt}")


def test_gemm_fp8_prefill_shape_sampled():
    # 70B FFN prefill shape: m 2048, k 8192, n 28672, block 32, E8M0; sampled rows and columns
    w = synth.c4_weight()
    wd = bf16_dev(w)
    cd, sd = mx.mx_quantize_fp8(wd, 32, "e8m0")
    del wd
    cols = np.array([0, 1, 255, 256, 5000, 14335, 20000, 28671])
    rows = np.array([0, 1, 127, 128, 700, 1500, 2047])
    rc, rs = oracle.quantize_fp8(w[cols], 32, "e8m0")
    np.testing.assert_array_equal(to_host_bits(cd[cols]), rc)
    np.testing.assert_array_equal(to_host_bits(sd[cols]), rs)
    x = synth.c4_x()
    y = mx.mx_gemm_fp8(bf16_dev(x), cd, sd, 32, "e8m0", out_dtype=torch.float32)
    torch.cuda.synchronize()
    yref, aref = oracle.gemm_fp8(x[rows], rc, rs, 32, "e8m0")
    assert_gemm_close(to_host_bits(y[rows][:, cols]), yref, aref, False, "w8 prefill")


def test_gemm_fp8_generic_path():
    # k % 32 != 0: one thread per output
    m, n, k = 5, 33, 72
    x = synth.normal((m, k), "bf16", "g8g.x", 1.0)
    w = synth.normal((n, k), "bf16", "g8g.w", 0.02)
    rc, rs = oracle.quantize_fp8(w, 8, "e8m0")
    y = mx.mx_gemm_fp8(bf16_dev(x), torch.from_numpy(rc).to(DEV), torch.from_numpy(rs).to(DEV), 8, "e8m0",
                       out_dtype=torch.float32)
    torch.cuda.synchronize()
    yref, aref = oracle.gemm_fp8(x, rc, rs, 8, "e8m0")
    assert_gemm_close(to_host_bits(y), yref, aref, False, "w8 generic")


def test_fallback_scenario_sigma_below_1e4():
    # a sigma = 5e-5 layer: FP4 with E4M3 block scales flushes every block to zero, which the
    # fallback rule catches.  FP8 elements divide the block maximum by 448, so their scale must
    # reach lower still: E4M3 and UE5M3 scales flush this tensor too, E8M0 scales keep it
    w = synth.normal((64, 4096), "bf16", "fb.w", 5e-5)
    wd = bf16_dev(w)
    sigma = float(mx.mx_tensor_stats(wd).cpu().numpy()[1])
    assert mx.mx_use_fp8(sigma) and oracle.use_fp8(sigma)
    c4, s4 = mx.mx_quantize(wd, 32, "e4m3")
    assert torch.count_nonzero(s4).item() == 0  # every FP4 block flushed
    _, s8u, _, _ = check_quant(w, 32, "ue5m3")
    assert torch.count_nonzero(s8u).item() == 0
    c8, s8, _, _ = check_quant(w, 32, "e8m0")
    y8 = mx.mx_dequantize_fp8(c8, s8, 32, "e8m0", out_dtype=torch.float32).cpu().numpy().astype(np.float64)
    wf = synth.bf16_to_f32(w).astype(np.float64)
    assert np.mean((y8 - wf) ** 2) < 1e-2 * np.mean(wf ** 2)  # FP4 lost all of it (ratio 1)


def test_gemm_fp8_decode_shape_sampled():
    # decode GEMV shape: m 1, k 4096, n 14336, block 32, E8M0, sampled columns against the oracle
    x = synth.c3_x(1)
    w = synth.c3_weight(14336)
    wd = bf16_dev(w)
    cd, sd = mx.mx_quantize_fp8(wd, 32, "e8m0")
    cols = np.array([0, 1, 777, 8191, 14335])
    rc, rs = oracle.quantize_fp8(w[cols], 32, "e8m0")
    np.testing.assert_array_equal(to_host_bits(cd[cols]), rc)
    y = mx.mx_gemm_fp8(bf16_dev(x), cd, sd, 32, "e8m0", out_dtype=torch.float32)
    torch.cuda.synchronize()
    yref, aref = oracle.gemm_fp8(x, rc, rs, 32, "e8m0")
    assert_gemm_close(to_host_bits(y)[:, cols], yref, aref, False, "w8 decode")


def _decision_point_tensor(fmt, scale_bytes):
    """bf16 blocks of 32 whose maximum is 448 s (the block scale is then exactly s) and whose
    other elements are the bf16 values at and around s times every E4M3 decision point (the
    midpoints between neighbouring values), both signs."""
    table = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    mids = (table[:-1] + table[1:]) / 2
    blocks = []
    for sb in scale_bytes:
        s = oracle.scale_value(sb, fmt)
        t = (mids * s).astype(np.float32)
        bits = (t.view(np.uint32) >> 16).astype(np.int64)  # bf16 at or just below, then neighbours
        cand = np.concatenate([bits - 1, bits, bits + 1, bits + 2])
        vals = (cand.astype(np.uint32) << 16).view(np.float32)
        vals = vals[(vals > 0) & (vals <= 448 * s)]
        vals = np.where(np.arange(vals.size) % 2 == 0, vals, -vals).astype(np.float32)
        pad = (-vals.size) % 31
        vals = np.concatenate([vals, np.zeros(pad, dtype=np.float32)]).reshape(-1, 31)
        top = np.full((vals.shape[0], 1), 448 * s, dtype=np.float32)
        blocks.append(np.concatenate([top, vals], axis=1))
    x = np.concatenate(blocks).reshape(-1)
    pad = (-x.size) % 1024
    x = np.concatenate([x, np.zeros(pad, dtype=np.float32)]).reshape(-1, 1024)
    b = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.bf16_to_f32(b), x)  # every value is a bf16 value
    return b


@pytest.mark.parametrize("fmt,scale_bytes", [
    ("e4m3", [8 * e + m for e in range(1, 13) for m in range(8)]),
    ("ue5m3", [8 * e + m for e in range(6, 20) for m in range(8)]),
    ("e8m0", list(range(100, 140))),
])
def test_quantize_fp8_every_decision_point(fmt, scale_bytes):
    # exact decisions of the bf16 / g == 1 fast path at every E4M3 midpoint for every scale
    # mantissa (E4M3, UE5M3) and a range of powers of two (E8M0)
    x = _decision_point_tensor(fmt, scale_bytes)
    check_quant(x, 32, fmt)
