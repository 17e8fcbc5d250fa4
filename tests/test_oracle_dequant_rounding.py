"""Oracle pins: the output rounding of dequantization (hotelren.com/news/2192771, article
"量化技术演进与微缩量化原理", section 3.1 item 3: value = FP4 element x FP8 block scale x
per-tensor scale).  The dequantized value is one fp32 round-to-nearest-even of the exact
product e*s*g, and bf16 output is the nearest-even bf16 of that fp32 value.

Pinned against references that do not go through the oracle's own arithmetic:
 * fp32 -> bf16 (ox_f32_to_bf16): torch's float32 -> bfloat16 conversion on every fp32 bit
   pattern within +-4 ulps of every bf16 rounding midpoint (normal and subnormal, both signs),
   the largest finite values, zeros and infinities, and a random sweep of bit patterns;
 * fp32 rounding of e*s*g for tensor scales that are not powers of two: exact rational
   products (fractions) rounded to fp32 by an integer round-half-even written here, for every
   code and every finite non-zero scale byte of the three formats; bf16 output then through
   torch's conversion of that fp32 value;
 * the same for the FP8 weight fallback's dequantize (E4M3 elements).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

FMTS = ["e4m3", "ue5m3", "e8m0"]
G_VALUES = [0.37, 1.0 / 3.0, 3.3e-3, 1234.5]


def torch_bf16_bits(f32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def oracle_bf16_bits(ox, f32: np.ndarray) -> np.ndarray:
    return np.array([ox.f32_to_bf16(float(v)) for v in f32], dtype=np.uint16)


def test_f32_to_bf16_around_every_midpoint(ox):
    # a bf16 rounding midpoint is an fp32 pattern whose low 16 bits are 0x8000
    hi = np.arange(0, 0x7F80, dtype=np.uint32)  # every finite positive bf16 (incl. subnormals)
    mid = (hi << 16) | 0x8000
    offs = np.arange(-4, 5, dtype=np.int64)
    pats = (mid[:, None].astype(np.int64) + offs[None, :]).ravel().astype(np.uint32)
    pats = np.concatenate([pats, pats | 0x80000000])
    f = pats.view(np.float32)
    f = f[np.isfinite(f)]
    got = oracle_bf16_bits(ox, f)
    np.testing.assert_array_equal(got, torch_bf16_bits(f))


def test_f32_to_bf16_random_and_special(ox):
    rng = np.random.default_rng(2024)
    pats = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    special = np.array([0x00000000, 0x80000000, 0x7F7FFFFF, 0xFF7FFFFF, 0x7F7F8000, 0x7F7F7FFF,
                        0x7F7F8001, 0x7F800000, 0xFF800000, 0x00000001, 0x80000001, 0x00008000,
                        0x00018000, 0x007FFFFF, 0x00800000], dtype=np.uint32)
    f = np.concatenate([pats, special]).view(np.float32)
    fin = ~np.isnan(f)
    got = oracle_bf16_bits(ox, f[fin])
    np.testing.assert_array_equal(got, torch_bf16_bits(f[fin]))
    # NaN stays NaN (quiet): exponent all ones, mantissa non-zero
    for p in (0x7FC00000, 0x7F800001, 0xFFFFFFFF):
        b = ox.f32_to_bf16(float(np.array([p], dtype=np.uint32).view(np.float32)[0]))
        assert (b & 0x7F80) == 0x7F80 and (b & 0x7F) != 0


def f32_round_exact(q: Fraction) -> np.float32:
    """Nearest-even fp32 of an exact rational (written out: exponent, integer significand,
    Python's round-half-even on the significand; overflow to infinity)."""
    if q == 0:
        return np.float32(0.0)
    neg = q < 0
    a = -q if neg else q
    e = a.numerator.bit_length() - a.denominator.bit_length()  # 2^e <= a < 2^(e+2)
    if a < Fraction(2) ** e:
        e -= 1
    elif a >= Fraction(2) ** (e + 1):
        e += 1
    ue = max(e, -126) - 23  # the ulp of the binade (subnormal binade below 2^-126)
    sig = round(a / Fraction(2) ** ue)  # Fraction.__round__: nearest, ties to even
    if sig * Fraction(2) ** ue >= Fraction(2) ** 128:
        v = np.float32(np.inf)
    else:
        v = np.float32(float(sig) * 2.0 ** ue)  # sig <= 2^24: exact in double and fp32
        assert Fraction(float(v)) == sig * Fraction(2) ** ue
    return -v if neg else v


def _finite_scale_bytes(ox, fmt):
    out = []
    for b in range(256):
        s = ox.scale_value(b, fmt)
        if not np.isnan(s) and s > 0:
            out.append(b)
    return out


def _all_code_rows(nbytes):
    """rows x 16 packed code bytes: each row holds the 16 codes twice (32 elements)."""
    c = np.arange(16, dtype=np.uint8)
    el = np.concatenate([c, c[::-1]])  # 32 elements, every code in both nibble positions
    packed = (el[0::2] | (el[1::2] << 4)).astype(np.uint8)
    return np.tile(packed, (nbytes, 1)), el


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("g", G_VALUES)
def test_dequantize_rounding_non_power_of_two_g(ox, fmt, g):
    g32 = float(np.float32(g))
    sbytes = _finite_scale_bytes(ox, fmt)
    codes, el = _all_code_rows(len(sbytes))
    scales = np.array(sbytes, dtype=np.uint8)[:, None]
    got = ox.dequantize(codes, scales, 32, 32, fmt, g32, "f32")
    got_bf = ox.dequantize(codes, scales, 32, 32, fmt, g32, "bf16")
    e2m1 = [0, Fraction(1, 2), 1, Fraction(3, 2), 2, 3, 4, 6]
    gf = Fraction(g32)
    exp = np.empty_like(got)
    inexact = 0
    for r, sb in enumerate(sbytes):
        s = Fraction(ox.scale_value(sb, fmt))
        for j, c in enumerate(el):
            mag = e2m1[c & 7] * s * gf
            exp[r, j] = f32_round_exact(-mag if c & 8 else mag)
            if c == 8:
                exp[r, j] = np.float32(-0.0)
            inexact += np.isfinite(exp[r, j]) and Fraction(float(abs(exp[r, j]))) != mag
    np.testing.assert_array_equal(got.view(np.uint32), exp.view(np.uint32))
    np.testing.assert_array_equal(got_bf, torch_bf16_bits(exp.ravel()).reshape(exp.shape))
    # the fp32 rounding is exercised, not only exact products (1234.5 has 12 significant bits,
    # so its products are exact except where they underflow into fp32 subnormals)
    if g != 1234.5:
        assert inexact > 0


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("g", G_VALUES)
def test_dequantize_fp8_rounding_non_power_of_two_g(ox, fmt, g):
    g32 = float(np.float32(g))
    sbytes = _finite_scale_bytes(ox, fmt)[::3]  # every third scale byte, all element bytes
    elems = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    # 254 element bytes and two zero bytes per row: one block of 256 under one scale byte
    codes = np.tile(elems, (len(sbytes), 1))
    codes = np.concatenate([codes, np.zeros((len(sbytes), 2), dtype=np.uint8)], axis=1)
    scales = np.array(sbytes, dtype=np.uint8)[:, None]
    got = ox.dequantize_fp8(codes, scales, 256, fmt, g32, "f32")
    got_bf = ox.dequantize_fp8(codes, scales, 256, fmt, g32, "bf16")
    gf = Fraction(g32)
    e4m3 = [Fraction(torch.tensor([c], dtype=torch.uint8).view(torch.float8_e4m3fn).float().item())
            if c not in (0x7F, 0xFF) else None for c in range(256)]
    exp = np.empty_like(got)
    for r, sb in enumerate(sbytes):
        s = Fraction(ox.scale_value(sb, fmt))
        for j, c in enumerate(codes[r]):
            v = f32_round_exact(e4m3[c] * s * gf)
            exp[r, j] = -v if (c & 0x80) and v == 0 else v
    np.testing.assert_array_equal(got.view(np.uint32), exp.view(np.uint32))
    np.testing.assert_array_equal(got_bf, torch_bf16_bits(exp.ravel()).reshape(exp.shape))


def test_f32_round_exact_reference():
    """The rounding reference above against numpy's own double -> float32 conversion on values
    exactly representable in double (numpy rounds those once, to nearest even)."""
    rng = np.random.default_rng(5)
    d = rng.standard_normal(3000) * np.exp(rng.uniform(-110, 90, 3000))
    d = np.concatenate([d, [2.0 ** -149, 3 * 2.0 ** -151, 2.0 ** -150, 2.0 ** -151 * 5,
                            (2 - 2.0 ** -24) * 2.0 ** 127, (2 - 2.0 ** -23) * 2.0 ** 127, 1 + 2.0 ** -24,
                            1 + 3 * 2.0 ** -24]])
    for v in d:
        ref = np.float32(v)
        got = f32_round_exact(Fraction(float(v)))
        assert got.view(np.uint32) == ref.view(np.uint32), (v, got, ref)
