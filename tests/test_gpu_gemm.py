"""GPU parity: mx_gemm (W4A16 and W4A4) through the C ABI against the fp64 CPU oracle.

Tolerance (fixed by the benchmark spec for the matmul): |Y - Yref| <= 2e-5 * sum_k |x_k w_k|
on the fp32 output; bf16 output adds half a bf16 ulp of Yref (its own rounding).  Cases:
decode GEMV M in {1, 4, 16} and prefill GEMM with ragged M/N/K tails for every block size
and format, the generic path, k = 0, W4A4 (activation pre-pass bit-identical to
mx_quantize, then block-scaled FP4 MFMA), and the full-size workloads -- tiny round trip,
decode shapes, 70B-FFN prefill, 405B-FFN with two-level scaling -- on sampled outputs.
"""
import numpy as np
import pytest
import torch

import microscaling_fp4_weight_amd as mx
import oracle
import oracle_pool
import synth
from gpu_util import DEV, assert_gemm_close, bf16_dev, f32_dev, padding_positions, tiled_positions, to_host_bits

pytestmark = pytest.mark.gpu

FMTS = ["e4m3", "ue5m3", "e8m0"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mx.lib()


def quantize_ref(w, block, fmt, g=1.0):
    """Oracle weight quantization -> host arrays and device copies."""
    c, s = oracle.quantize(w, block, fmt, g)
    return c, s, torch.from_numpy(c).to(DEV), torch.from_numpy(s).to(DEV)


def check(x, c, s, cd, sd, block, fmt, g, mode, out, rows=None, cols=None, what=""):
    xd = bf16_dev(x)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    y = mx.mx_gemm(xd, cd, sd, block, fmt, g, mode, out_dtype=dt)
    torch.cuda.synchronize()
    yref, aref = oracle.gemm(x, c, s, block, fmt, g, mode, mrows=rows, ncols=cols)
    got = to_host_bits(y.float())
    if rows is not None:
        got = got[rows]
    if cols is not None:
        got = got[:, cols]
    assert_gemm_close(got, yref, aref, out == "bf16", what or f"{mode} {fmt} B={block} {out}")
    return y


@pytest.mark.parametrize("m", [1, 4, 16])
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("block", [4, 8, 16, 32, 64, 128, 256])
def test_gemv_a16(m, fmt, block):
    n, k = 100, 768  # ragged n; k = 6 k-tiles, split over 4 waves unevenly
    x = synth.normal((m, k), "bf16", f"gv.x.{m}", 1.0)
    w = synth.normal((n, k), "bf16", "gv.w", 0.02, 0.01, 20.0)
    c, s, cd, sd = quantize_ref(w, block, fmt)
    for out in ("f32", "bf16"):
        check(x, c, s, cd, sd, block, fmt, 1.0, "a16", out)


# m <= 2 with block 32 and k in {4096, 8192, 16384} on short streams takes the sweeping GEMV
# (a grid of at most 1024 workgroups, up to 4 steps each, over 8 KB units of codes): one and
# several steps, workgroups with different step counts (unit counts just past 1024), rows
# per unit 4, 2 and 1, one and two rows of X.  For m = 1 the preshuffled layout must give
# bit-identical results.
@pytest.mark.parametrize("m", [1, 2])
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k", [(1000, 4096), (8000, 4096), (2050, 8192), (777, 16384), (4096, 16384)])
def test_gemv_sweep(fmt, n, k, m):
    g = float(np.float32(0.37)) if fmt != "e8m0" else 1.0
    x = synth.normal((m, k), "bf16", f"sw.x.{k}.{m}", 1.0)
    w = synth.normal((n, k), "bf16", f"sw.w.{n}.{k}", 0.02, 0.01, 20.0)
    c, s, cd, sd = quantize_ref(w, 32, fmt, g)
    yr = {}
    for out in ("f32", "bf16"):
        yr[out] = check(x, c, s, cd, sd, 32, fmt, g, "a16", out, what=f"sweep m={m} {fmt} {n}x{k} {out}")
    if m > 1:
        return
    cp, sp = mx.mx_quantize(bf16_dev(w), 32, fmt, g, layout="preshuffled")
    for out, dt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
        yp = mx.mx_gemm(bf16_dev(x), cp, sp, 32, fmt, g, "a16", out_dtype=dt, layout="preshuffled")
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_host_bits(yp), to_host_bits(yr[out]))


# The 2 <= m <= 16 decode GEMV with k = 4096 (16-row weight units streamed by LDS-DMA, X in
# registers): every block size it takes and every format, m at the edges and in between, n with
# a ragged last unit, a grid with one unit per workgroup (n 100) and one with several (n 16 *
# 2100 + 9: 2101 units over 526 workgroups), g != 1 for E4M3 / UE5M3; fp32 and bf16 out.
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("block", [32, 64, 128, 256])
@pytest.mark.parametrize("m,n", [(3, 100), (16, 100), (5, 33609), (16, 33609)])
def test_gemv16(fmt, block, m, n):
    k = 4096
    g = float(np.float32(0.37)) if fmt != "e8m0" else 1.0
    x = synth.normal((m, k), "bf16", f"g16.x.{m}", 1.0)
    w = synth.normal((n, k), "bf16", f"g16.w.{n}", 0.02, 0.01, 20.0)
    c, s, cd, sd = quantize_ref(w, block, fmt, g)
    cols = None if n <= 100 else np.unique(np.concatenate([np.arange(0, n, 37), np.arange(n - 40, n)]))
    c_sel, s_sel = (c, s) if cols is None else (c[cols], s[cols])
    xd = bf16_dev(x)
    for out, dt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
        y = mx.mx_gemm(xd, cd, sd, block, fmt, g, "a16", out_dtype=dt)
        torch.cuda.synchronize()
        yref, aref = oracle.gemm(x, c_sel, s_sel, block, fmt, g, "a16")
        got = to_host_bits(y.float())
        if cols is not None:
            got = got[:, cols]
        assert_gemm_close(got, yref, aref, out == "bf16", f"gemv16 m={m} n={n} {fmt} B={block} {out}")


# Row strides through the small-m kernels: activation rows longer than k (16-byte aligned, which
# the 2 <= m <= 16 kernel takes, and unaligned, which goes to the generic GEMV) and output rows
# longer than n, whose extra columns must stay untouched; m = 1 takes the sweeping kernel
# (n 1000) and the row-group kernel (n 33609).
@pytest.mark.parametrize("ldx", [4096 + 64, 4096 + 3])
@pytest.mark.parametrize("m,n", [(1, 1000), (1, 33609), (2, 1000), (7, 1000), (16, 33609)])
def test_gemv_small_m_strides(ldx, m, n):
    k, fmt = 4096, "ue5m3"
    g = float(np.float32(0.37))
    x = synth.normal((m, ldx), "bf16", f"gvs.x.{m}.{ldx}", 1.0)
    w = synth.normal((n, k), "bf16", f"gvs.w.{n}", 0.02, 0.01, 20.0)
    c, s, cd, sd = quantize_ref(w, 32, fmt, g)
    cols = np.unique(np.concatenate([np.arange(0, n, 97), np.arange(n - 20, n)]))
    yref, aref = oracle.gemm(np.ascontiguousarray(x[:, :k]), c[cols], s[cols], 32, fmt, g, "a16")
    xd = bf16_dev(x)[:, :k]
    for dt in (torch.float32, torch.bfloat16):
        big = torch.full((m, n + 24), float("nan"), dtype=dt, device=DEV)
        y = big[:, :n]
        mx.mx_gemm(xd, cd, sd, 32, fmt, g, "a16", y=y)
        torch.cuda.synchronize()
        got = to_host_bits(y.float())[:, cols]
        assert_gemm_close(got, yref, aref, dt == torch.bfloat16, f"strided GEMV m={m} n={n} ldx={ldx} {dt}")
        assert torch.isnan(big[:, n:].float()).all()


# Zero-scale blocks through the GEMVs (an E4M3 / UE5M3 scale's mantissa multiplies each block's
# sum there, so a zero scale must give a zero block): all-zero blocks and blocks small enough
# to flush (a <= 3 s_min: 1e-4 under E4M3, 1e-6 under UE5M3), on the sweeping kernel (k 4096)
# and the row kernel (k 768), one and two rows of X; m 300 takes the tile kernels (k 4096: the
# wide-tile one for E4M3 / UE5M3, the 128 x 256 one for E8M0; k 768: the unpipelined one).
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k", [(96, 4096), (100, 768)])
@pytest.mark.parametrize("m", [1, 2, 300])
def test_gemv_zero_and_flushed_blocks(fmt, n, k, m):
    g = float(np.float32(0.37)) if fmt != "e8m0" else 1.0
    x = synth.normal((m, k), "bf16", f"gz.x.{m}.{k}", 1.0)
    w32 = synth.normal((n, k), "f32", f"gz.w.{n}.{k}", 0.02)
    blocks = w32.reshape(n, k // 32, 32)
    blocks[::3, ::5] = 0.0                                   # all-zero blocks
    tiny = 1e-4 if fmt == "e4m3" else 1e-6
    blocks[1::3, 1::4] *= tiny / 0.02 / 4                     # flushing blocks (|x| < tiny)
    w = torch.from_numpy(blocks.reshape(n, k)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    c, s, cd, sd = quantize_ref(w, 32, fmt, g)
    assert (s == 0).any()
    for out in ("f32", "bf16"):
        check(x, c, s, cd, sd, 32, fmt, g, "a16", out, what=f"zero blocks m={m} {fmt} {n}x{k} {out}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("block", [4, 16, 32, 128])
def test_gemm_a16_ragged(fmt, block):
    m, n, k = 200, 300, 640  # 2 x 3 workgroup tiles, all ragged; k-tail of 128
    x = synth.normal((m, k), "bf16", "gg.x", 1.0)
    w = synth.normal((n, k), "bf16", "gg.w", 0.02, 0.01, 20.0)
    c, s, cd, sd = quantize_ref(w, block, fmt)
    for out in ("f32", "bf16"):
        check(x, c, s, cd, sd, block, fmt, 1.0, "a16", out)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("mnk", [(200, 300, 1024), (17, 256, 512), (300, 520, 2048), (256, 512, 1536),
                                 (500, 1948, 512), (1024, 2048, 512)])
def test_gemm_a16_pipelined(fmt, mnk):
    """Block 32 and k a multiple of 512: the pipelined kernel (128 x 256 tiles, 3-stage LDS
    ring, 512-k scale windows) -- ragged m and n, one to several scale windows; the last two
    shapes (m-tiles a multiple of 4, n-tiles of 8) take the XCD-grouped tile order, one and
    two groups of m-tiles, the first with ragged m and n."""
    m, n, k = mnk
    x = synth.normal((m, k), "bf16", f"gp.x.{m}", 1.0)
    w = synth.normal((n, k), "bf16", f"gp.w.{n}", 0.02, 0.01, 20.0)
    c, s, cd, sd = quantize_ref(w, 32, fmt)
    for out in ("f32", "bf16"):
        check(x, c, s, cd, sd, 32, fmt, 1.0, "a16", out)


@pytest.mark.parametrize("fmt", ["e8m0", "ue5m3"])
@pytest.mark.parametrize("ldy", [600, 523])
def test_gemm_a16_strided_output(fmt, ldy):
    """Output rows with a stride beyond n, 16-byte aligned (chunk epilogue) or odd (element
    epilogue), through the 128 x 256 kernel (E8M0 here) and the wide-tile one (UE5M3); the
    columns past n must stay untouched."""
    g = float(np.float32(0.37)) if fmt != "e8m0" else 1.0
    m, n, k = 300, 520, 1024
    x = synth.normal((m, k), "bf16", "gst.x", 1.0)
    w = synth.normal((n, k), "bf16", "gst.w", 0.02, 0.01, 20.0)
    c, s = oracle.quantize(w, 32, fmt, g)
    cd, sd = torch.from_numpy(c).to(DEV), torch.from_numpy(s).to(DEV)
    yref, aref = oracle.gemm(x, c, s, 32, fmt, g, "a16")
    for dt in (torch.float32, torch.bfloat16):
        big = torch.full((m, ldy), float("nan"), dtype=dt, device=DEV)
        y = big[:, :n]
        mx.mx_gemm(bf16_dev(x), cd, sd, 32, fmt, g, "a16", y=y)
        torch.cuda.synchronize()
        assert_gemm_close(to_host_bits(y.float()), yref, aref, dt == torch.bfloat16, f"strided y {fmt} {ldy} {dt}")
        assert torch.isnan(big[:, n:].float()).all()


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_a16_pipelined_tensor_scale_and_stride(fmt):
    """Two-level scaling (g != 1) and an activation row stride larger than k."""
    m, n, k, g = 130, 260, 1024, float(np.float32(0.37))
    x = synth.normal((m, k + 64), "bf16", "gps.x", 1.0)
    w = synth.normal((n, k), "bf16", "gps.w", 0.05)
    c, s = oracle.quantize(w, 32, fmt, g)
    cd, sd = torch.from_numpy(c).to(DEV), torch.from_numpy(s).to(DEV)
    xd = bf16_dev(x)[:, :k]
    y = mx.mx_gemm(xd, cd, sd, 32, fmt, g, "a16", out_dtype=torch.float32)
    torch.cuda.synchronize()
    yref, aref = oracle.gemm(np.ascontiguousarray(x[:, :k]), c, s, 32, fmt, g, "a16")
    assert_gemm_close(to_host_bits(y), yref, aref, False, f"a16 pipelined g {fmt}")


def test_gemm_a16_k_tail_32():
    m, n, k = 40, 70, 160  # k % 128 == 32
    x = synth.normal((m, k), "bf16", "gt.x", 1.0)
    w = synth.normal((n, k), "bf16", "gt.w", 0.02)
    for m_ in (5, 40):
        c, s, cd, sd = quantize_ref(w, 32, "e8m0")
        check(x[:m_], c, s, cd, sd, 32, "e8m0", 1.0, "a16", "f32")


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_tensor_scale(fmt):
    g = float(np.float32(0.0173))
    m, n, k = 33, 64, 256
    x = synth.normal((m, k), "bf16", "gs.x", 1.0)
    w = synth.normal((n, k), "bf16", "gs.w", 0.02, 0.01, 20.0)
    c, s, cd, sd = quantize_ref(w, 32, fmt, g)
    check(x, c, s, cd, sd, 32, fmt, g, "a16", "f32")
    check(x[:3], c, s, cd, sd, 32, fmt, g, "a16", "bf16")


def test_gemm_generic_path():
    # k = 48 is not a multiple of 32: the generic kernel; an odd activation stride too
    m, n, k = 7, 9, 48
    x = synth.normal((m, k), "bf16", "gp.x", 1.0)
    w = synth.normal((n, k), "bf16", "gp.w", 0.02)
    for fmt in FMTS:
        c, s, cd, sd = quantize_ref(w, 16, fmt)
        check(x, c, s, cd, sd, 16, fmt, 1.0, "a16", "f32")
    big = synth.normal((m, 75), "bf16", "gp.ld", 1.0)
    xd = bf16_dev(big)[:, :64]
    w2 = synth.normal((n, 64), "bf16", "gp.w2", 0.02)
    c, s, cd, sd = quantize_ref(w2, 32, "e8m0")
    y = mx.mx_gemm(xd, cd, sd, 32, "e8m0", 1.0, "a16", out_dtype=torch.float32)
    yref, aref = oracle.gemm(np.ascontiguousarray(big[:, :64]), c, s, 32, "e8m0")
    assert_gemm_close(to_host_bits(y), yref, aref, False, "strided x")


def test_gemm_k_zero_writes_zeros():
    x = torch.empty((3, 0), dtype=torch.bfloat16, device=DEV)
    cd = torch.empty((5, 0), dtype=torch.uint8, device=DEV)
    sd = torch.empty((5, 0), dtype=torch.uint8, device=DEV)
    y = torch.full((3, 5), 7.0, dtype=torch.float32, device=DEV)
    mx.mx_gemm(x, cd, sd, 32, "e8m0", 1.0, "a16", y=y)
    assert torch.count_nonzero(y).item() == 0


@pytest.mark.parametrize("mnk", [(1, 64, 128), (16, 96, 256), (200, 300, 640), (129, 257, 160)])
def test_gemm_a4(mnk):
    m, n, k = mnk
    x = synth.normal((m, k), "bf16", f"ga.x.{m}", 1.0)
    w = synth.normal((n, k), "bf16", "ga.w", 0.015, 0.001, 20.0)
    c, s, cd, sd = quantize_ref(w, 32, "e8m0")
    for out in ("f32", "bf16"):
        check(x, c, s, cd, sd, 32, "e8m0", 1.0, "a4", out)


@pytest.mark.parametrize("layout", ["rowmajor", "tiled"])
@pytest.mark.parametrize("ldy", [600, 523])
def test_gemm_a4_strided_output(layout, ldy):
    """W4A4 into output rows with a stride beyond n (16-byte aligned: chunk epilogue; odd:
    element epilogue), row-major and tiled weight scales; the columns past n stay untouched."""
    m, n, k = 300, 520, 1024
    x = synth.normal((m, k), "bf16", "gsa.x", 1.0)
    w = synth.normal((n, k), "bf16", "gsa.w", 0.015, 0.001, 20.0)
    c, s = oracle.quantize(w, 32, "e8m0")
    cd, sd = mx.mx_quantize(bf16_dev(w), 32, "e8m0", layout=layout)
    np.testing.assert_array_equal(to_host_bits(cd), c)
    yref, aref = oracle.gemm(x, c, s, 32, "e8m0", 1.0, "a4")
    for dt in (torch.float32, torch.bfloat16):
        big = torch.full((m, ldy), float("nan"), dtype=dt, device=DEV)
        y = big[:, :n]
        mx.mx_gemm(bf16_dev(x), cd, sd, 32, "e8m0", 1.0, "a4", y=y, layout=layout)
        torch.cuda.synchronize()
        assert_gemm_close(to_host_bits(y.float()), yref, aref, dt == torch.bfloat16, f"a4 strided y {layout} {ldy} {dt}")
        assert torch.isnan(big[:, n:].float()).all()


@pytest.mark.parametrize("k", [512, 4224, 160])
def test_gemm_a4_prepass_matches_quantize(k):
    """The activations quantized inside mx_gemm (workspace) are byte-identical to
    mx_quantize(X, 32, E8M0) and to the oracle.  With k % 128 == 0 the matrix-core kernel
    runs and the workspace holds the scales in the tiled layout (mx_quantize with
    layout "tiled"); otherwise row-major."""
    m, n = 37, 64
    x = synth.normal((m, k), "bf16", f"gw.x.{k}", 1.0, 0.01, 20.0)
    w = synth.normal((n, k), "bf16", "gw.w", 0.02)
    c, s, cd, sd = quantize_ref(w, 32, "e8m0")
    xd = bf16_dev(x)
    need = mx.mx_gemm_workspace_size(m, n, k, 32, "a4")
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    mx.mx_gemm(xd, cd, sd, 32, "e8m0", 1.0, "a4", workspace=ws)
    torch.cuda.synchronize()
    wsh = to_host_bits(ws)
    codes = wsh[: m * k // 2].reshape(m, k // 2)
    off = (m * k // 2 + 255) // 256 * 256
    rc, rs = oracle.quantize(x, 32, "e8m0")
    np.testing.assert_array_equal(codes, rc)
    qc, _ = mx.mx_quantize(xd, 32, "e8m0")
    np.testing.assert_array_equal(to_host_bits(qc), codes)
    wsc = wsh[off:]
    if k % 128 == 0:
        np.testing.assert_array_equal(wsc[tiled_positions(m, k)], rs)
        assert np.all(wsc[padding_positions(m, k)] == 0)
    else:
        np.testing.assert_array_equal(wsc[: m * k // 32].reshape(m, k // 32), rs)


# ------------------------------------------------------------------------ full-size workloads

def test_c1_tiny_round_trip_and_gemv():
    """256 x 256 fp32 weight ~ N(0, 0.02^2) with 1% outliers x20, block 32 E4M3, g = 1:
    quantize -> dequantize bit-exact; y = W^ x within tolerance; error split reported."""
    w = synth.c1_weight()
    x = synth.c1_x()
    c, s = mx.mx_quantize(f32_dev(w), 32, "e4m3")
    rc, rs = oracle.quantize(w, 32, "e4m3")
    np.testing.assert_array_equal(to_host_bits(c), rc)
    np.testing.assert_array_equal(to_host_bits(s), rs)
    y = mx.mx_dequantize(c, s, 256, 32, "e4m3", out_dtype=torch.float32)
    np.testing.assert_array_equal(to_host_bits(y).view(np.uint32),
                                  oracle.dequantize(rc, rs, 256, 32, "e4m3").view(np.uint32))
    for out in ("f32", "bf16"):
        check(x, rc, rs, c, s, 32, "e4m3", 1.0, "a16", out, what=f"C1 gemv {out}")
    split = oracle.mse_split(w, 32, "e4m3")
    assert split["total"] > 0


@pytest.mark.parametrize("n", [4096, 14336])
def test_c3_decode_gemv(n):
    """Decode GEMV K=4096, N in {4096, 14336}, M in {1, 4, 16}; block 32 E8M0; bf16 out.  The
    whole weight's codes and scales bit-exact, and every output of every M checked."""
    w = synth.c3_weight(n)
    wd = bf16_dev(w)
    del w
    cd, sd = mx.mx_quantize(wd, 32, "e8m0")
    gemms = [(m, list(range(m)), "a16") for m in (1, 4, 16)]
    rc, rs, ys = oracle_pool.full_weight(f"c3.{n}", n, "e8m0", 1.0, gemms)
    np.testing.assert_array_equal(to_host_bits(cd), rc)
    np.testing.assert_array_equal(to_host_bits(sd), rs)
    for (m, _, _), (yref, aref) in zip(gemms, ys):
        x = synth.c3_x(m)
        for dt in (torch.bfloat16, torch.float32):
            y = mx.mx_gemm(bf16_dev(x), cd, sd, 32, "e8m0", 1.0, "a16", out_dtype=dt)
            torch.cuda.synchronize()
            assert_gemm_close(to_host_bits(y.float()), yref, aref, dt == torch.bfloat16, f"C3 n={n} m={m} {dt}")


# one activation row in each 256-row m-tile of the 70B-FFN prefill (first and last rows included)
C4_ROWS = [0, 293, 586, 879, 1172, 1465, 1758, 2047]


@pytest.fixture(scope="module")
def c4_full():
    """The 70B-FFN weight quantized on the GPU (row-major and tiled scales) and by the oracle
    (all 28672 rows, over host processes), with the oracle's W4A16 and W4A4 products for the
    C4_ROWS activation rows against every weight row."""
    w = synth.c4_weight()
    wd = bf16_dev(w)
    del w
    cd, sd = mx.mx_quantize(wd, 32, "e8m0")
    _, sdt = mx.mx_quantize(wd, 32, "e8m0", layout="tiled")
    del wd
    torch.cuda.empty_cache()
    rc, rs, ys = oracle_pool.full_weight("c4", 28672, "e8m0", 1.0,
                                         [(2048, C4_ROWS, "a16"), (2048, C4_ROWS, "a4")])
    np.testing.assert_array_equal(to_host_bits(cd), rc)
    np.testing.assert_array_equal(to_host_bits(sd), rs)
    return cd, sd, sdt, {"a16": ys[0], "a4": ys[1]}


@pytest.mark.parametrize("mode,layout", [("a16", "rowmajor"), ("a4", "rowmajor"), ("a4", "tiled")])
def test_c4_prefill(mode, layout, c4_full):
    """70B FFN prefill M=2048, K=8192, N=28672, block 32 E8M0: W4A16 and W4A4 (row-major and
    tiled weight scales); all 28672 columns of one row in each 256-row m-tile, so every output
    tile (and the W4A4 half tiles of the last round) is reached; fp32 and bf16 out."""
    cd, sd, sdt, ref = c4_full
    yref, aref = ref[mode]
    xd = bf16_dev(synth.c4_x())
    for dt in (torch.float32, torch.bfloat16):
        y = mx.mx_gemm(xd, cd, sdt if layout == "tiled" else sd, 32, "e8m0", 1.0, mode, out_dtype=dt,
                       layout=layout)
        torch.cuda.synchronize()
        assert_gemm_close(to_host_bits(y[C4_ROWS].float()), yref, aref, dt == torch.bfloat16,
                          f"C4 {mode} {layout} {dt}")
        del y


# The one-workgroup-per-CU W4A16 kernels at a shape the small tests never reach: m 200, n 28600
# (E8M0: 224 tiles of 128 x 256, too few for the two-workgroup kernel -> the 8-wave 128 x 256
# kernel; E4M3 / UE5M3: the 8-wave 256 x 256 kernel, 112 tiles), the last n-tile ragged.
# Sampled rows and columns.
@pytest.mark.parametrize("fmt,g", [("e8m0", 1.0), ("ue5m3", 0.37), ("e4m3", 1.0)])
def test_gemm_a16_wide_tiles_sampled(fmt, g):
    g = float(np.float32(g))
    m, n, k = 200, 28600, 1024
    x = synth.normal((m, k), "bf16", "gw.x", 1.0)
    w = synth.normal((n, k), "bf16", "gw.w", 0.02, 0.01, 20.0)
    wd = bf16_dev(w)
    cd, sd = mx.mx_quantize(wd, 32, fmt, g)
    del wd
    cols = np.array([0, 1, 255, 256, 9999, 28415, 28416, 28599])
    rows = np.array([0, 1, 31, 32, 127, 128, 199])
    rc, rs = oracle.quantize(w[cols], 32, fmt, g)
    np.testing.assert_array_equal(to_host_bits(cd[cols]), rc)
    np.testing.assert_array_equal(to_host_bits(sd[cols]), rs)
    for dt in (torch.float32, torch.bfloat16):
        y = mx.mx_gemm(bf16_dev(x), cd, sd, 32, fmt, g, "a16", out_dtype=dt)
        torch.cuda.synchronize()
        yref, aref = oracle.gemm(x[rows], rc, rs, 32, fmt, g, "a16")
        assert_gemm_close(to_host_bits(y[rows][:, cols].float()), yref, aref, dt == torch.bfloat16,
                          f"wide tiles {fmt} {dt}")


# The two-workgroup W4A16 kernel (E8M0 scales, more 128 x 256 tiles than CUs; 4 waves of 64 x 128)
# over its three tile orders: m 1000 x n 16300 (the XCD-grouped order), m 300 x n 28600 (n-tiles
# by XCD), m 260 x n 33000 (plain order); m and n ragged in each, k from two 256-k scale windows
# to eight, g = 1 and g != 1, both output types, and output rows with a stride beyond n
# (16-byte aligned: chunk epilogue; odd: element epilogue) whose columns past n must stay
# untouched; m 1000 x n 20400 (640 tiles) leaves its last round a quarter full.  The same cases
# with E4M3 / UE5M3 scales run the 8-wave 256 x 256 kernel (m > 128) over its tile orders.  Sampled rows and columns: both sides of every wave block and tile edge
# that the sample reaches.
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m,n,k,g,ldy_extra", [(1000, 16300, 1024, 0.37, 0), (300, 28600, 512, 1.0, 8),
                                               (260, 33000, 2048, 1.0, 3), (1000, 20400, 1024, 1.0, 8)])
def test_gemm_a16_paired_sampled(m, n, k, g, ldy_extra, fmt):
    g = float(np.float32(g))
    x = synth.normal((m, k), "bf16", f"gq.x.{m}", 1.0)
    w = synth.normal((n, k), "bf16", f"gq.w.{n}", 0.02, 0.01, 20.0)
    wd = bf16_dev(w)
    cd, sd = mx.mx_quantize(wd, 32, fmt, g)
    del wd
    last = (n - 1) // 256 * 256
    cols = np.unique(np.array([0, 1, 63, 64, 127, 128, 255, 256, 383, 384, n // 2, last - 1, last, last + 127,
                               last + 128, n - 1]))
    cols = cols[cols < n]
    rows = np.unique(np.array([0, 1, 63, 64, 127, 128, 191, 255, 256, m // 2, m - 1]))
    rows = rows[rows < m]
    rc, rs = oracle.quantize(w[cols], 32, fmt, g)
    np.testing.assert_array_equal(to_host_bits(cd[cols]), rc)
    np.testing.assert_array_equal(to_host_bits(sd[cols]), rs)
    yref, aref = oracle.gemm(x[rows], rc, rs, 32, fmt, g, "a16")
    xd = bf16_dev(x)
    for dt in (torch.float32, torch.bfloat16):
        if ldy_extra:
            big = torch.full((m, n + ldy_extra), float("nan"), dtype=dt, device=DEV)
            y = big[:, :n]
            mx.mx_gemm(xd, cd, sd, 32, fmt, g, "a16", y=y)
        else:
            y = mx.mx_gemm(xd, cd, sd, 32, fmt, g, "a16", out_dtype=dt)
        torch.cuda.synchronize()
        assert_gemm_close(to_host_bits(y[rows][:, cols].float()), yref, aref, dt == torch.bfloat16,
                          f"paired {fmt} {m}x{n}x{k} {dt}")
        if ldy_extra:
            assert torch.isnan(big[:, n:].float()).all()
        del y


# activation rows of the 405B-FFN products: one in each 256-row m-tile for m = 4096
C5_ROWS = {1: [0], 256: [0, 85, 170, 255], 4096: [256 * i + (97 * i) % 256 for i in range(15)] + [4095]}


@pytest.fixture(scope="module")
def c5_weights():
    """The 405B-FFN weight (53248 x 16384, UE5M3 block 32, per-tensor g) quantized on the GPU and,
    all rows, by the oracle over host processes, with the oracle's products for C5_ROWS."""
    w = synth.c5_weight()
    g = synth.c5_tensor_scale(w)
    wd = bf16_dev(w)
    del w
    cd, sd = mx.mx_quantize(wd, 32, "ue5m3", g)
    del wd
    torch.cuda.empty_cache()
    gemms = [(m, C5_ROWS[m], "a16") for m in (1, 256, 4096)]
    rc, rs, ys = oracle_pool.full_weight("c5", 53248, "ue5m3", g, gemms)
    np.testing.assert_array_equal(to_host_bits(cd), rc)
    np.testing.assert_array_equal(to_host_bits(sd), rs)
    return cd, sd, g, {m: y for (m, _, _), y in zip(gemms, ys)}


@pytest.mark.parametrize("m", [1, 256, 4096])
def test_c5_two_level(m, c5_weights):
    """405B FFN K=16384, N=53248, UE5M3 block 32 with per-tensor g; W4A16, fp32 accumulate,
    bf16 out (fp32 out also for M=1): every column of the sampled rows (all 53248 outputs for
    M=1, one row per 256-row m-tile for M=4096)."""
    cd, sd, g, ref = c5_weights
    yref, aref = ref[m]
    rows = C5_ROWS[m]
    xd = bf16_dev(synth.c5_x(m))
    for out in (("f32", "bf16") if m == 1 else ("bf16",)):
        dt = torch.float32 if out == "f32" else torch.bfloat16
        y = mx.mx_gemm(xd, cd, sd, 32, "ue5m3", g, "a16", out_dtype=dt)
        torch.cuda.synchronize()
        assert_gemm_close(to_host_bits(y[rows].float()), yref, aref, out == "bf16", f"C5 m={m} {out}")
        del y


def test_gemv_rows_past_2gb_stride():
    """Activation rows so far apart that they span more than 2^31 bytes (3.2 / 4.3 GB): the
    GEMV kernels address X with 32-bit offsets, so such a call must take the 64-bit path and
    still agree with the oracle (m = 4 and 16, both outputs)."""
    n, k = 96, 512
    w = synth.normal((n, k), "bf16", "span.w", 0.02)
    c, s, cd, sd = quantize_ref(w, 32, "e8m0")
    for m, ld in ((4, 1 << 29), (16, 1 << 27)):
        assert ((m - 1) * ld + k) * 2 >= 1 << 31
        x = synth.normal((m, k), "bf16", f"span.x.{m}", 1.0)
        print(f"span test m={m} ld={ld}", flush=True)
        buf = torch.zeros((m - 1) * ld + k, dtype=torch.bfloat16, device=DEV)
        xs = buf.as_strided((m, k), (ld, 1))
        xs.copy_(bf16_dev(x))
        for out in ("f32", "bf16"):
            dt = torch.float32 if out == "f32" else torch.bfloat16
            y = mx.mx_gemm(xs, cd, sd, 32, "e8m0", 1.0, "a16", out_dtype=dt)
            torch.cuda.synchronize()
            yref, aref = oracle.gemm(x, c, s, 32, "e8m0", 1.0, "a16")
            assert_gemm_close(to_host_bits(y.float()), yref, aref, out == "bf16", f"span m={m} {out}")
        del buf, xs
        torch.cuda.empty_cache()
