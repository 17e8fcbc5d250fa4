"""Oracle pins: the FP8 weight fallback of hotelren.com/news/2192771 (article
"量化技术演进与微缩量化原理", section 5.3 item 1: sigma < 1e-4 layers go to FP8; section 6 item 1:
key layers in FP8), read as E4M3 elements (OCP E4M3FN) in the same blocks under the same scale
formats, block scale nearest to absmax / (448 g).

 * element decode of all 256 bytes against torch's float8_e4m3fn;
 * element rounding with a unit scale against torch's own fp32 -> float8_e4m3fn conversion
   (round to nearest even) for every bf16 magnitude below the saturation point, and with
   power-of-two scales against the same conversion of the exactly rescaled value;
 * element and scale rounding for non-power-of-two scales and per-tensor g against brute
   force in exact rational arithmetic (fractions), dense around the midpoints;
 * saturation at 448, sign and zero handling, flush of a zero scale;
 * quantize / dequantize round trip of representable (code, scale) pairs and the GEMM against
   numpy's float64 product of the dequantized weights;
 * the fallback test itself: sigma < 1e-4.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

FMTS = ["e4m3", "ue5m3", "e8m0"]


def e4m3_table():
    return [Fraction(np.float64(torch.tensor([c], dtype=torch.uint8).view(torch.float8_e4m3fn).float().item()))
            for c in range(0x7F)]


def test_element_decode_all_bytes(ox):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = np.array([ox.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2  # 0x7F, 0xFF
    assert np.array_equal(got[~nan], ref[~nan])
    assert ox.e4m3_value(0x7E) == 448.0 and ox.e4m3_value(1) == 2.0 ** -9


def test_rounding_unit_scale_vs_torch(ox):
    # every positive bf16 value below 464 (the midpoint past 448), and their negatives
    bits = np.arange(1, 0x43E8, dtype=np.uint32)
    v = (bits << 16).view(np.float32)
    v = np.concatenate([v, -v]).astype(np.float32)
    got = ox.elem_codes_fp8(v.astype(np.float64), 1.0, 1.0)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("e", [-20, -9, -3, 0, 5, 30])
def test_rounding_pow2_scales_vs_torch(ox, e):
    rng = np.random.default_rng(100 + e)
    s = 2.0 ** e
    v = (rng.standard_normal(20000) * 60).astype(np.float32)
    v = v[np.abs(v) < 460]
    x = (v.astype(np.float64) * s).astype(np.float32)  # exact rescale (no under/overflow here)
    assert np.array_equal(x.astype(np.float64) / s, v.astype(np.float64))
    got = ox.elem_codes_fp8(x.astype(np.float64), s, 1.0)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def brute_elem(x: float, s: float, g: float, table) -> int:
    q = abs(Fraction(x)) / (Fraction(s) * Fraction(g))
    best, bd = None, None
    for c, v in enumerate(table):
        d = abs(v - q)
        if bd is None or d < bd or (d == bd and c % 2 == 0):
            best, bd = c, d
    return best | (0x80 if np.signbit(x) else 0)


@pytest.mark.parametrize("fmt", ["e4m3", "ue5m3"])
def test_rounding_general_scales_brute_force(ox, fmt):
    table = e4m3_table()
    rng = np.random.default_rng(7)
    for trial in range(12):
        sb = int(rng.integers(0x30, 0x60))
        s = ox.scale_value(sb, fmt)
        g = float(np.float32(rng.uniform(0.3, 3.0))) if trial % 2 else 1.0
        # points at, just around and between the decision midpoints, and random ones
        mids = [(table[i] + table[i + 1]) / 2 for i in range(len(table) - 1)]
        xs = []
        for mdl in mids[::7]:
            t = float(mdl * Fraction(s) * Fraction(g))
            xs += [t, np.nextafter(t, 0.0), np.nextafter(t, np.inf)]
        xs += list(rng.standard_normal(200) * 100 * s * g)
        xs = [float(np.float32(v)) for v in xs]
        got = ox.elem_codes_fp8(np.array(xs), s, g)
        for x, c in zip(xs, got):
            assert c == brute_elem(x, s, g, table), (x, s, g)


@pytest.mark.parametrize("fmt", FMTS)
def test_scale_rounding_brute_force(ox, fmt):
    vals = [(Fraction(ox.scale_value(c, fmt)), c) for c in range(256)
            if np.isfinite(ox.scale_value(c, fmt)) and ox.scale_value(c, fmt) >= 0
            and not (fmt == "e4m3" and c >= 0x80)]
    vals.sort()
    rng = np.random.default_rng(3)
    a = np.concatenate([np.exp(rng.uniform(-60, 60, 300)), [0.0, 1e-45, 3e38]])
    for g in (1.0, float(np.float32(0.37))):
        got = ox.scale_bytes_fp8(a, g, fmt)
        for av, c in zip(a, got):
            q = Fraction(float(av)) / (448 * Fraction(g))
            best = min(vals, key=lambda t: (abs(t[0] - q), -t[0] if fmt == "e8m0" else t[1] % 2))
            assert c == best[1], (av, g, fmt)


def test_saturation_sign_zero(ox):
    assert ox.elem_code_fp8(500.0, 1.0) == 0x7E and ox.elem_code_fp8(-1e30, 1.0) == 0xFE
    assert ox.elem_code_fp8(-0.0, 1.0) == 0x80 and ox.elem_code_fp8(0.0, 1.0) == 0x00
    assert ox.elem_code_fp8(-3.0, 0.0) == 0x80  # zero scale flushes, sign kept
    assert ox.elem_code_fp8(2.0 ** -10, 1.0) == 0x00  # tie at half the smallest subnormal -> even 0
    assert ox.elem_code_fp8(3 * 2.0 ** -11, 1.0) == 0x01


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("block", [4, 32, 256])
def test_round_trip_representable(ox, fmt, block):
    rng = np.random.default_rng(block)
    rows, k = 8, 512
    table = np.array([ox.e4m3_value(c) for c in range(0x7F)])
    sbytes = {"e4m3": (0x20, 0x50), "ue5m3": (0x60, 0x90), "e8m0": (110, 135)}[fmt]
    x = np.empty((rows, k), dtype=np.float32)
    for r in range(rows):
        for b in range(k // block):
            s = ox.scale_value(int(rng.integers(*sbytes)), fmt)
            blk = rng.choice(table, block) * np.where(rng.random(block) < 0.5, -1, 1)
            blk[int(rng.integers(block))] = 448.0  # the block maximum fixes the scale at s
            x[r, b * block:(b + 1) * block] = blk * s
    c, s = ox.quantize_fp8(x, block, fmt)
    y = ox.dequantize_fp8(c, s, block, fmt)
    assert np.array_equal(y, x)


def test_gemm_fp8_vs_numpy(ox, syn):
    x = syn.normal((5, 256), "bf16", "fp8.x", 1.0)
    w = syn.normal((40, 256), "f32", "fp8.w", 0.02, 0.01, 20.0)
    c, s = ox.quantize_fp8(w, 32, "ue5m3")
    wd = ox.dequantize_fp8(c, s, 32, "ue5m3").astype(np.float64)
    xf = syn.bf16_to_f32(x).astype(np.float64)
    y, a = ox.gemm_fp8(x, c, s, 32, "ue5m3")
    assert np.allclose(y, xf @ wd.T, rtol=1e-13, atol=1e-15)
    assert np.allclose(a, np.abs(xf) @ np.abs(wd).T, rtol=1e-13)
    # FP8 keeps far more of the weight than FP4 on the same tensor (3 mantissa bits against 1)
    c4, s4 = ox.quantize(w, 32, "ue5m3")
    w4 = ox.dequantize(c4, s4, 256, 32, "ue5m3").astype(np.float64)
    assert np.mean((wd - w) ** 2) < 0.1 * np.mean((w4 - w) ** 2)


def test_fallback_rule(ox):
    assert ox.use_fp8(5e-5) and ox.use_fp8(0.0)
    assert not ox.use_fp8(1e-4) and not ox.use_fp8(0.02)
