"""GPU parity: mx_quantize / mx_dequantize through the C ABI against the CPU oracle.

Codes and scale bytes must be bit-exact; dequantized values bit-exact.  Cases: every block
size x scale format x input dtype on small tensors spanning several workgroups with a
ragged tail; the edge-case tensor (every scale byte, every bf16 magnitude to 6, exact ties,
zero / flush / saturating / subnormal blocks); shapes that take the generic path (k not a
multiple of 32, odd row stride); empty tensors; a per-tensor scale; every E4M3 / UE5M3 scale
mantissa with every bf16 magnitude under it; and the full-size Llama-7B FFN (4096 x 11008)
and 405B FFN (53248 x 16384) weights in the launch configuration the benchmark times, whole
tensors compared.
"""
import numpy as np
import pytest
import torch

import microscaling_fp4_weight_amd as mx
import oracle
import oracle_pool
import synth
from gpu_util import DEV, bf16_dev, edge_tensor, f32_dev, to_host_bits

pytestmark = pytest.mark.gpu

FMTS = ["e4m3", "ue5m3", "e8m0"]
BLOCKS = [4, 8, 16, 32, 64, 128, 256]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mx.lib()


def run_quant(x_host: np.ndarray, block: int, fmt: str, g: float = 1.0):
    xd = bf16_dev(x_host) if x_host.dtype == np.uint16 else f32_dev(x_host)
    c, s = mx.mx_quantize(xd, block, fmt, g)
    torch.cuda.synchronize()
    return to_host_bits(c), to_host_bits(s)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("block", BLOCKS)
def test_quantize_small(dtype, fmt, block):
    # 37 rows x 1280: 1480 lanes of 32 elements -> 6 workgroups, the last one partial
    x = synth.normal((37, 1280), dtype, f"gq.{dtype}", 0.02, 0.01, 20.0)
    c, s = run_quant(x, block, fmt)
    rc, rs = oracle.quantize(x, block, fmt)
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(c, rc)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("block", BLOCKS)
def test_quantize_edge_tensor(fmt, block):
    x = edge_tensor()
    c, s = run_quant(x, block, fmt)
    rc, rs = oracle.quantize(x, block, fmt)
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(c, rc)
    # and as fp32 input
    xf = synth.bf16_to_f32(x)
    c2, s2 = run_quant(xf, block, fmt)
    np.testing.assert_array_equal(s2, rs)
    np.testing.assert_array_equal(c2, rc)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("g", [0.37, 2.0 ** -7, 1234.5])
def test_quantize_tensor_scale(fmt, g):
    g = float(np.float32(g))
    x = synth.normal((19, 1024), "bf16", "gq.g", 0.3, 0.01, 20.0)
    x = np.concatenate([x, edge_tensor(1024)[:40]])
    xf = synth.bf16_to_f32(x)
    for block in (4, 8, 16, 32, 64, 128, 256):
        rc, rs = oracle.quantize(x, block, fmt, g)
        for inp in (x, xf):  # bf16 input, and the same values as fp32
            c, s = run_quant(inp, block, fmt, g)
            np.testing.assert_array_equal(s, rs)
            np.testing.assert_array_equal(c, rc)


def _tensor_scale_decision_blocks(fmt: str, g: float, dtype: str) -> np.ndarray:
    """Blocks of 32, rows of 1024: for every positive finite scale byte s of `fmt` under the
    per-tensor scale g, a block maximum a = 6 s g and, around each decision point t s' g
    (s' the scale the oracle gives that maximum; t = 0.25, 0.75, ..., 5), fp32 values at
    0, +-1, ..., +-40 fp32 units (f32) or the four nearest bf16 values (bf16), both signs."""
    amax = []
    for byte in range(256):
        sv = oracle.scale_value(byte, fmt)
        if not np.isfinite(sv) or sv <= 0:
            continue
        if 6.0 * sv * g > 3.0e38:
            continue
        a = np.float32(6.0 * sv * g)
        if dtype == "bf16" and np.isfinite(a):  # nearest bf16 (ties to even)
            ab = np.array([a], dtype=np.float32).view(np.uint32).astype(np.uint64)
            ab = (ab + 0x7FFF + ((ab >> 16) & 1)) >> 16 << 16
            a = ab.astype(np.uint32).view(np.float32)[0]
        if not np.isfinite(a) or a < 1e-38:
            continue
        amax.append(a)
    amax = np.array(amax, dtype=np.float32)
    probe = np.zeros((amax.size, 32), dtype=np.float32)
    probe[:, 0] = amax
    _, sb = oracle.quantize(probe, 32, fmt, g)
    ts = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    offs = np.array([0, 1, -1, 2, -2, 3, -3, 5, -5, 8, -8, 12, -12, 15, -15, 16, -16, 17, -17, 20, -20,
                     30, -30, 40, -40], dtype=np.int64)
    blocks = []
    for a, byte in zip(amax, sb[:, 0]):
        sv = oracle.scale_value(int(byte), fmt)
        pts = (ts * sv * g).astype(np.float32)
        bits = pts.view(np.uint32).astype(np.int64)
        if dtype == "f32":
            cand = (bits[:, None] + offs[None, :]).ravel()
        else:
            hb = bits >> 16
            cand = (np.concatenate([hb - 1, hb, hb + 1, hb + 2]) << 16)
        cand = cand[(cand > 0) & (cand < 0x7F800000)].astype(np.uint32)
        vals = cand.view(np.float32)
        vals = vals[vals <= a]
        vals = np.where(np.arange(vals.size) % 2 == 0, vals, -vals).astype(np.float32)
        pad = (-vals.size) % 31
        vals = np.concatenate([vals, np.zeros(pad, dtype=np.float32)]).reshape(-1, 31)
        top = np.full((vals.shape[0], 1), a, dtype=np.float32)
        blocks.append(np.concatenate([top, vals], axis=1))
    x = np.concatenate(blocks).reshape(-1)
    x = np.concatenate([x, np.zeros((-x.size) % 1024, dtype=np.float32)]).reshape(-1, 1024)
    if dtype == "bf16":
        b = (x.view(np.uint32) >> 16).astype(np.uint16)
        assert np.array_equal(synth.bf16_to_f32(b), x)  # every value is a bf16 value
        return b
    return x


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("g", [0.37, 1.0 / 3.0, 0.70710677, 3.3e-3, 1234.5, 2.0 ** -7, 4.0, 2e-38, 1e37])
def test_quantize_tensor_scale_decision_points(dtype, fmt, g):
    # with g != 1 the kernel compares each |x| with the block's seven decision thresholds t s g,
    # rounded to fp32 bit patterns; they come from a per-workgroup table of the eight scale
    # mantissas scaled by the block's power of two, or, where that would leave the normal fp32
    # range (the smallest and largest scales, and every block at g = 2e-38 or 1e37), from fp64
    # products.  These blocks put elements at and around every decision point of every scale,
    # so both ways are exercised against the exact oracle
    g = float(np.float32(g))
    x = _tensor_scale_decision_blocks(fmt, g, dtype)
    c, s = run_quant(x, 32, fmt, g)
    rc, rs = oracle.quantize(x, 32, fmt, g)
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(c, rc)


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_generic_path(fmt):
    # k = 48 (not a multiple of 32) and an odd row stride both take the generic kernel
    x = synth.normal((33, 48), "bf16", "gq.gen", 0.05, 0.01, 20.0)
    for block in (4, 8, 16):
        c, s = run_quant(x, block, fmt)
        rc, rs = oracle.quantize(x, block, fmt)
        np.testing.assert_array_equal(s, rs)
        np.testing.assert_array_equal(c, rc)
    big = synth.normal((9, 263), "bf16", "gq.ld", 0.05, 0.01, 20.0)
    xd = bf16_dev(big)[:, :256]  # row stride 263 elements
    c, s = mx.mx_quantize(xd, 32, fmt)
    rc, rs = oracle.quantize(np.ascontiguousarray(big[:, :256]), 32, fmt)
    np.testing.assert_array_equal(to_host_bits(s), rs)
    np.testing.assert_array_equal(to_host_bits(c), rc)


def test_quantize_empty():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    c, s = mx.mx_quantize(x, 32, "e8m0")
    assert c.shape == (0, 32) and s.shape == (0, 2)


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("block", [4, 16, 32, 128])
@pytest.mark.parametrize("g", [1.0, 0.37])
def test_dequantize(out, fmt, block, g):
    g = float(np.float32(g))
    x = np.concatenate([synth.normal((21, 512), "bf16", "gd", 0.02, 0.01, 20.0), edge_tensor(512)[:64]])
    rc, rs = oracle.quantize(x, block, fmt, g)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    y = mx.mx_dequantize(torch.from_numpy(rc).to(DEV), torch.from_numpy(rs).to(DEV), 512, block,
                         fmt, g, out_dtype=dt)
    ref = oracle.dequantize(rc, rs, 512, block, fmt, g, out)
    got = to_host_bits(y)
    if out == "f32":
        np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))
    else:
        np.testing.assert_array_equal(got, ref)


def test_dequantize_all_scale_bytes():
    # every code with every finite scale byte (including those whose products overflow); the
    # formats' NaN bytes are left out because the library's contract (include/mx.h) leaves
    # their decoded value unspecified: mx_quantize never writes them
    for fmt in FMTS:
        codes = np.tile(np.arange(256, dtype=np.uint8), 256).reshape(256, 256)  # 512 elems/row
        scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 512 // 32, axis=1)
        ok = np.array([np.isfinite(oracle.scale_value(b, fmt)) for b in range(256)])
        codes, scales = codes[ok], scales[ok]
        for out in ("f32", "bf16"):
            dt = torch.float32 if out == "f32" else torch.bfloat16
            y = mx.mx_dequantize(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV),
                                 512, 32, fmt, 1.0, out_dtype=dt)
            ref = oracle.dequantize(codes, scales, 512, 32, fmt, 1.0, out)
            got = to_host_bits(y)
            if out == "f32":
                np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))
            else:
                np.testing.assert_array_equal(got, ref)


def test_quantize_deterministic():
    x = synth.normal((64, 4096), "bf16", "gq.det", 0.02, 0.01, 20.0)
    xd = bf16_dev(x)
    a = [to_host_bits(t) for t in mx.mx_quantize(xd, 16, "ue5m3")]
    b = [to_host_bits(t) for t in mx.mx_quantize(xd, 16, "ue5m3")]
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


SAMPLE_ROWS_C2 = [0, 1, 777, 2048, 3001, 4094, 4095]


@pytest.mark.parametrize("sigma", synth.C2_SIGMAS)
def test_c2_full_size_sampled(sigma):
    """Llama-7B FFN weight 4096 x 11008 bf16, every block size and format, as the benchmark
    launches it; rows compared with the oracle on a sample."""
    w = synth.c2_weight(sigma)
    wd = bf16_dev(w)
    for fmt in FMTS:
        for block in BLOCKS:
            c, s = mx.mx_quantize(wd, block, fmt)
            rows = SAMPLE_ROWS_C2
            rc, rs = oracle.quantize(w[rows], block, fmt)
            np.testing.assert_array_equal(to_host_bits(s[rows]), rs, err_msg=f"{fmt} B={block}")
            np.testing.assert_array_equal(to_host_bits(c[rows]), rc, err_msg=f"{fmt} B={block}")
            y = mx.mx_dequantize(c, s, 11008, block, fmt, 1.0, out_dtype=torch.bfloat16)
            np.testing.assert_array_equal(to_host_bits(y[rows]),
                                          oracle.dequantize(rc, rs, 11008, block, fmt, 1.0, "bf16"))
    del wd


C2_FULL_CASES = [(0.02, 32, "e8m0"), (0.02, 32, "e4m3"), (0.02, 32, "ue5m3"), (0.02, 4, "e4m3"),
                 (0.02, 256, "ue5m3"), (0.005, 32, "e8m0"), (0.1, 32, "e8m0")]


@pytest.mark.parametrize("sigma,block,fmt", C2_FULL_CASES)
def test_c2_full_tensor_exact(sigma, block, fmt):
    """The whole Llama-7B FFN weight (4096 x 11008 bf16, 45 M elements), in the launch the
    benchmark times: every code byte, scale byte and dequantized bf16 element equal to the
    oracle's -- the block-32 E8M0 quantize is the benchmark's dominant kernel."""
    w = synth.c2_weight(sigma)
    wd = bf16_dev(w)
    c, s = mx.mx_quantize(wd, block, fmt)
    y = mx.mx_dequantize(c, s, 11008, block, fmt, 1.0, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    del wd
    rc, rs = oracle.quantize(w, block, fmt)
    np.testing.assert_array_equal(to_host_bits(s), rs, err_msg=f"scales {fmt} B={block}")
    np.testing.assert_array_equal(to_host_bits(c), rc, err_msg=f"codes {fmt} B={block}")
    np.testing.assert_array_equal(to_host_bits(y), oracle.dequantize(rc, rs, 11008, block, fmt, 1.0, "bf16"),
                                  err_msg=f"dequantized {fmt} B={block}")


def test_c5_full_tensor_two_level():
    """405B FFN weight 53248 x 16384 bf16, UE5M3 block 32 times a per-tensor scale
    g = fl32(max|W| / (6 * 114688)): every code and scale byte of the whole tensor equal to the
    oracle's (oracle over host processes); dequantized rows sampled, including the narrow bands."""
    w = synth.c5_weight()
    g = synth.c5_tensor_scale(w)
    wd = bf16_dev(w)
    c, s = mx.mx_quantize(wd, 32, "ue5m3", g)
    del wd
    torch.cuda.synchronize()
    rc, rs, _ = oracle_pool.full_weight("c5", 53248, "ue5m3", g, [])
    np.testing.assert_array_equal(to_host_bits(s), rs)
    np.testing.assert_array_equal(to_host_bits(c), rc)
    rows = [0, 3327, 3328 * 3, 3328 * 3 + 17, 26000, 3328 * 15, 53247]
    y = mx.mx_dequantize(c[rows].contiguous(), s[rows].contiguous(), 16384, 32, "ue5m3", g,
                         out_dtype=torch.bfloat16)
    np.testing.assert_array_equal(to_host_bits(y), oracle.dequantize(rc[rows], rs[rows], 16384, 32, "ue5m3", g, "bf16"))


def _mantissa_blocks(fmt: str, dtype: str) -> np.ndarray:
    """Blocks of 32 whose maximum is 6 s (so the block scale is exactly s) for every scale
    mantissa at three normal exponents and every subnormal scale of the format, holding every
    bf16 magnitude up to 6 s with both signs, and (fp32 input) the fp32 values within 64 ulps
    of every decision point t s of the element rounding."""
    exps = {"e4m3": (-6, 0, 5), "ue5m3": (-14, 0, 10)}[fmt]
    smin_exp = {"e4m3": -9, "ue5m3": -17}[fmt]
    scales = [(1 + mi / 8) * 2.0 ** e for mi in range(8) for e in exps]
    scales += [mi * 2.0 ** smin_exp for mi in range(1, 8)]
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    out = []
    for sc in scales:
        top = np.float32(6.0 * sc)
        assert float(top) == 6.0 * sc and (np.array([top]).view(np.uint32)[0] & 0xFFFF) == 0  # bf16-exact
        hi = int(np.array([top]).view(np.uint32)[0] >> 16)
        mags = (np.arange(1, hi + 1, dtype=np.uint32) << 16).view(np.float32)
        vals = [mags, -mags, np.array([0.0, -0.0], dtype=np.float32)]
        if dtype == "f32":
            for t in ties:
                b = np.array([np.float32(t * sc)]).view(np.uint32).astype(np.int64)[0]
                near = np.arange(b - 64, b + 65, dtype=np.int64).astype(np.uint32).view(np.float32)
                vals += [near, -near]
        v = np.concatenate(vals)
        v = v[np.abs(v) <= top]
        nb = -(-len(v) // 31)
        v = np.pad(v, (0, nb * 31 - len(v)))
        blk = np.empty((nb, 32), dtype=np.float32)
        blk[:, 1:] = v.reshape(nb, 31)
        blk[:, 0] = np.where(np.arange(nb) % 2 == 0, top, -top)  # the maximum, alternating sign
        out.append(blk.reshape(-1))
    x = np.concatenate(out)
    pad = (-len(x)) % 512
    x = np.concatenate([x, np.zeros(pad, dtype=np.float32)]).reshape(-1, 512)
    if dtype == "bf16":
        return (x.view(np.uint32) >> 16).astype(np.uint16)  # exact: every value is bf16
    return x


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fmt", ["e4m3", "ue5m3"])
def test_quantize_every_scale_mantissa(fmt, dtype):
    """The element encode divides by a block scale with a mantissa (E4M3 / UE5M3): every code
    decided exactly for all eight mantissas (and the subnormal scales), g = 1, block 32."""
    x = _mantissa_blocks(fmt, dtype)
    c, s = run_quant(x, 32, fmt)
    rc, rs = oracle.quantize(x, 32, fmt)
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(c, rc)
