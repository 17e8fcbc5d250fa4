"""Oracle pins: the number formats.

The E2M1 table is checked against the printed grid (tests/golden/e2m1_grid.txt, with its
citations); E4M3 and E8M0 decoding against torch's float8_e4m3fn / float8_e8m0fnu (library
routines); UE5M3, which no library implements, against closed-form points and structure.
"""
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


def test_e2m1_table_matches_grid(ox):
    for code, value in _golden_rows("e2m1_grid.txt"):
        v = ox.e2m1_value(int(code))
        assert v == float(value), (code, v, value)
        assert math.copysign(1.0, v) == math.copysign(1.0, float(value))  # -0.0 for code 8


def test_e2m1_bit_layout(ox):
    # [sign][e1 e0][m]: the sign bit only flips the sign; e=0 is the subnormal pair {0, 0.5};
    # each exponent step doubles the value; the mantissa bit adds half.
    for c in range(8):
        assert ox.e2m1_value(c | 8) == -ox.e2m1_value(c)
    assert ox.e2m1_value(0b000) == 0.0 and ox.e2m1_value(0b001) == 0.5
    for e in (1, 2, 3):
        base = ox.e2m1_value(e << 1)
        assert base == 2.0 ** (e - 1)
        assert ox.e2m1_value((e << 1) | 1) == 1.5 * base
    assert max(ox.e2m1_value(c) for c in range(16)) == 6.0


def test_scale_golden_points(ox):
    for fmt, byte, value in _golden_rows("scale_formats.txt"):
        v = ox.scale_value(int(byte, 16), fmt)
        if value == "nan":
            assert math.isnan(v), (fmt, byte)
        else:
            assert v == float(value), (fmt, byte, v, value)


def test_e4m3_decode_matches_torch(ox):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(256):
        v = ox.scale_value(b, "e4m3")
        if math.isnan(ref[b]):
            assert math.isnan(v), b
        else:
            assert v == ref[b], (b, v, ref[b])


def test_e8m0_decode_matches_torch(ox):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    for b in range(256):
        v = ox.scale_value(b, "e8m0")
        if math.isnan(ref[b]):
            assert math.isnan(v), b
        else:
            assert v == ref[b], (b, v, ref[b])


def test_ue5m3_structure(ox):
    # Unsigned 5-bit exponent, 3-bit mantissa: 255 finite non-negative values, strictly
    # increasing with the byte; within a binade the step is 1/8 of the binade's base; the
    # subnormal range (exponent field 0) is evenly spaced at the smallest step.
    vals = [ox.scale_value(b, "ue5m3") for b in range(255)]
    assert all(vals[i] < vals[i + 1] for i in range(254))
    assert math.isnan(ox.scale_value(255, "ue5m3"))
    step = 2.0 ** -17
    for m in range(9):  # exponent field 0 (subnormal) and the first normal: evenly spaced
        assert vals[m] == m * step
    for e in range(1, 32):  # each binade doubles, and is split in 8 equal steps
        base = vals[e << 3]
        if e < 31:
            assert vals[(e + 1) << 3] == 2 * base
        for m in range(1, 8):
            b = (e << 3) | m
            if b < 255:
                assert vals[b] - vals[b - 1] == base / 8
    assert vals[0x78] == 1.0 and vals[254] == 114688.0
    # UE5M3 covers E4M3's whole positive range and more (the page's point of the format)
    assert vals[1] < ox.scale_value(1, "e4m3") and vals[254] > ox.scale_value(0x7E, "e4m3")
