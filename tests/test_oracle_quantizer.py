"""Oracle pins: properties of the block quantizer as a whole.

 * exact round trip: codes and scales that a quantizer could have produced (every block holds
   a +-6 code) survive dequantize -> quantize unchanged, including -0 codes and fp32-subnormal
   dequantized values;
 * idempotence: quantize o dequantize o quantize == quantize when every block's max code is +-6;
 * flush: all-zero blocks, and blocks whose absmax is at most 3 x the smallest non-zero scale
   (E4M3 / UE5M3), become zero; a tensor with sigma 1e-4 under E4M3 dequantizes to all zeros
   (hotelren.com/news/2192771 article, section 5.3 item 1: a layer with weight sigma < 1e-4
   comes out all zero);
 * saturation of the scale and clipping of elements at +-6;
 * layout: two codes per byte, even element in the low nibble; blocks run along k.
"""
import numpy as np
import pytest

FMTS = ["e4m3", "ue5m3", "e8m0"]


def _valid_scale_bytes(ox, fmt, g=1.0):
    """Non-zero, non-NaN scale bytes whose 6*s*g is finite in fp32."""
    out = []
    for b in range(256):
        s = ox.scale_value(b, fmt)
        if np.isnan(s) or s <= 0 or not np.isfinite(np.float32(6.0 * s * g)):
            continue
        out.append(b)
    return np.array(out, dtype=np.uint8)


def _random_codes(rng, rows, k, block):
    codes = rng.integers(0, 16, size=(rows, k), dtype=np.uint8)
    # one +-6 code per block at a random position
    nb = k // block
    pos = rng.integers(0, block, size=(rows, nb))
    sign = rng.integers(0, 2, size=(rows, nb)) * 8
    for r in range(rows):
        for b in range(nb):
            codes[r, b * block + pos[r, b]] = 7 | sign[r, b]
            blk = codes[r, b * block:(b + 1) * block]
            # no other element may exceed the max in magnitude; ties with 6 are fine
    return codes


def _pack(codes):
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("block", [4, 32, 256])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_round_trip(ox, fmt, block, out):
    rng = np.random.default_rng(block * 7 + len(fmt))
    sb = _valid_scale_bytes(ox, fmt)
    k = 512
    rows = (len(sb) * block + k - 1) // k + 1
    codes = _random_codes(rng, rows, k, block)
    scales = np.resize(sb, rows * (k // block)).reshape(rows, k // block)
    packed = _pack(codes)
    deq = ox.dequantize(packed, scales, k, block, fmt, 1.0, out)
    c2, s2 = ox.quantize(deq, block, fmt, 1.0)
    np.testing.assert_array_equal(s2, scales)
    np.testing.assert_array_equal(c2, packed)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("g", [0.25, 8.0])
def test_round_trip_power_of_two_tensor_scale(ox, fmt, g):
    rng = np.random.default_rng(11)
    block, k = 32, 256
    sb = _valid_scale_bytes(ox, fmt, g)
    rows = len(sb) * block // k + 1
    codes = _random_codes(rng, rows, k, block)
    scales = np.resize(sb, rows * (k // block)).reshape(rows, k // block)
    packed = _pack(codes)
    deq = ox.dequantize(packed, scales, k, block, fmt, g, "f32")
    c2, s2 = ox.quantize(deq, block, fmt, g)
    np.testing.assert_array_equal(s2, scales)
    np.testing.assert_array_equal(c2, packed)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("block", [4, 16, 64])
def test_idempotent(ox, syn, fmt, block):
    x = syn.normal((64, 1024), "bf16", "idem", 0.02, 0.01, 20.0)
    c1, s1 = ox.quantize(x, block, fmt)
    d1 = ox.dequantize(c1, s1, 1024, block, fmt, 1.0, "f32")
    c2, s2 = ox.quantize(d1, block, fmt)
    # blocks whose maximum element is coded +-6 are fixed points
    codes = np.stack([c1 & 15, c1 >> 4], axis=-1).reshape(64, 1024)
    has6 = ((codes.reshape(64, -1, block) & 7) == 7).any(axis=2)
    assert has6.mean() > 0.5
    np.testing.assert_array_equal(s2[has6], s1[has6])
    bytes_per_block = block // 2
    cb1 = c1.reshape(64, -1, bytes_per_block)[has6]
    cb2 = c2.reshape(64, -1, bytes_per_block)[has6]
    np.testing.assert_array_equal(cb2, cb1)


def test_layout_nibbles_and_blocks(ox):
    # x = [0.5, 1, 1.5, 2, 3, 4, 6, -6] repeated; E8M0 scale 1 (absmax 6 -> 6/6 = 1).
    vals = np.array([0.5, 1, 1.5, 2, 3, 4, 6, -6], dtype=np.float32)
    x = np.tile(vals, 4)[None, :]
    codes, scales = ox.quantize(x, 8, "e8m0")
    assert scales.tolist() == [[127, 127, 127, 127]]
    assert codes[0, :4].tolist() == [0x21, 0x43, 0x65, 0xF7]  # even element in the low nibble


def test_flush_all_zero_blocks(ox):
    x = np.zeros((2, 64), dtype=np.float32)
    x[1, 32:] = -0.0
    for fmt in FMTS:
        c, s = ox.quantize(x, 32, fmt)
        assert (s == 0).all()  # E4M3/UE5M3: zero scale; E8M0: the smallest scale 2^-127
        assert (c[0] == 0).all() and (c[1, :16] == 0).all() and (c[1, 16:] == 0x88).all()


@pytest.mark.parametrize("fmt,smin", [("e4m3", 2.0 ** -9), ("ue5m3", 2.0 ** -17)])
def test_flush_boundary(ox, fmt, smin):
    """A block flushes iff absmax <= 3 * smin (absmax/6 <= smin/2, the tie going to code 0)."""
    a = np.float32(3.0 * smin)
    assert ox.scale_byte(float(a), 1.0, fmt) == 0
    above = np.nextafter(a, np.float32(1.0))
    assert ox.scale_byte(float(above), 1.0, fmt) == 1
    x = np.full((1, 32), a, dtype=np.float32)
    c, s = ox.quantize(x, 32, fmt)
    assert s[0, 0] == 0 and (c == 0).all()


def test_sigma_1e4_e4m3_flushes_everything(ox, syn):
    x = syn.normal((128, 4096), "bf16", "tiny", 1e-4)
    c, s = ox.quantize(x, 32, "e4m3")
    deq = ox.dequantize(c, s, 4096, 32, "e4m3", 1.0, "f32")
    assert (s == 0).all() and not np.any(deq)
    # UE5M3's wider range keeps it
    c2, s2 = ox.quantize(x, 32, "ue5m3")
    assert (s2 > 0).all()


def test_scale_saturation_and_clip(ox):
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = 1e4
    x[0, 1] = -1e4
    x[0, 2] = 448.0 * 4.0
    c, s = ox.quantize(x, 32, "e4m3")
    assert s[0, 0] == 0x7E  # 448
    assert c[0, 0] == (7 | (15 << 4))  # +6 and -6
    assert c[0, 1] & 15 == 6  # 1792/448 = 4


def test_e8m0_scale_closed_form(ox):
    """E8M0 scale = 2^k nearest to a/6: k = floor(log2(a)) - 3 + [a >= 1.125 * 2^floor(log2 a)]
    (the midpoint 1.5 * 2^k of a/6 is a = 9 * 2^k)."""
    rng = np.random.default_rng(5)
    a = np.exp(rng.uniform(-80, 80, 200_000)).astype(np.float32).astype(np.float64)
    e = np.floor(np.log2(a))
    k = e - 3 + (a >= 1.125 * 2.0 ** e)
    want = np.clip(k + 127, 0, 254).astype(np.uint8)
    np.testing.assert_array_equal(ox.scale_bytes(a, 1.0, "e8m0"), want)
