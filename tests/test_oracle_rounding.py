"""Oracle pins: the two roundings (block scale onto FP8 / E8M0, element onto E2M1).

Each is checked against something other than the oracle's own midpoint search:
 * elements: brute-force argmin of |x - q*s*g| over the 8 magnitudes, ties to the even code,
   on every finite bf16 magnitude and on fp32 values packed around every tie;
 * E4M3 / E8M0 scales: torch's float8_e4m3fn / float8_e8m0fnu conversions (in their ranges);
 * UE5M3 scales: brute-force argmin over its 255 finite values.
It also checks the property the GPU scale path relies on: rounding the correctly rounded
fp32 quotient fl32(a/6) gives the same byte as rounding the exact a/6.
"""
import numpy as np
import pytest
import torch

E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def brute_e2m1(x: np.ndarray, s: float, g: float) -> np.ndarray:
    """argmin_j |x| - q_j*s*g| with ties to the even code, plus the sign bit (s > 0).
    Distances are exact in double for |x| < 64 s g; above that the nearest is 6 (code 7)."""
    big = np.abs(x) >= 64.0 * s * g
    ax = np.where(big, 0.0, np.abs(x))[:, None]
    d = np.abs(ax - E2M1_MAG[None, :] * (s * g))
    best = d.min(axis=1, keepdims=True)
    ties = d == best
    # lowest even index among the minima, else the lowest index
    even = ties & (np.arange(8)[None, :] % 2 == 0)
    idx = np.where(even.any(axis=1), even.argmax(axis=1), ties.argmax(axis=1))
    idx = np.where(big, 7, idx)
    return (idx | np.where(np.signbit(x), 8, 0)).astype(np.uint8)


def all_bf16_finite() -> np.ndarray:
    b = np.arange(65536, dtype=np.uint32)
    f = (b << 16).view(np.float32)
    return f[np.isfinite(f)].astype(np.float64)


def around(values, n_ulps: int) -> np.ndarray:
    """fp32 values within n_ulps of each given (positive) fp32 value."""
    out = []
    for v in values:
        b = np.array([v], dtype=np.float32).view(np.uint32)[0].astype(np.int64)
        bs = np.arange(max(b - n_ulps, 0), b + n_ulps + 1, dtype=np.int64).astype(np.uint32)
        out.append(bs.view(np.float32))
    return np.concatenate(out).astype(np.float64)


TIES = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
SCALES = [1.0, 2.0 ** -9, 1.125, 1.875 * 2.0 ** 3, 0.75 * 2.0 ** -8, 2.0 ** -127, 2.0 ** 120]


@pytest.mark.parametrize("s", SCALES)
def test_elem_code_all_bf16(ox, s):
    x = all_bf16_finite()
    got = ox.elem_codes(x, s, 1.0)
    np.testing.assert_array_equal(got, brute_e2m1(x, s, 1.0))


@pytest.mark.parametrize("s,g", [(1.0, 1.0), (1.5, 1.0), (1.875 * 2.0 ** -5, 1.0),
                                 (1.25, float(np.float32(0.3))), (2.0 ** -20, 1.0e3), (1.0, 2.0 ** -3)])
def test_elem_code_fp32_around_ties(ox, s, g):
    pts = [t * s * g for t in TIES] + [q * s * g for q in E2M1_MAG[1:]]
    x = around(pts, 300)
    x = np.concatenate([x, -x, [0.0, -0.0, 7.0 * s * g, 1e30 * s * g]])
    got = ox.elem_codes(x, s, g)
    if g == 1.0 or (g == 2.0 ** -3):  # products exact in double: brute force is exact too
        np.testing.assert_array_equal(got, brute_e2m1(x, s, g))
    else:  # compare through exact rationals
        from fractions import Fraction
        sg = Fraction(s) * Fraction(g)
        for xi, gi in zip(x[::37], got[::37]):
            d = [abs(abs(Fraction(xi)) - Fraction(q) * sg) for q in E2M1_MAG]
            best = min(d)
            cands = [j for j in range(8) if d[j] == best]
            j = next((c for c in cands if c % 2 == 0), cands[0])
            assert gi == (j | (8 if np.signbit(xi) else 0)), (xi, gi, j)


def test_elem_code_random_fp32(ox):
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(2_000_000) * rng.choice([0.1, 1.0, 4.0], 2_000_000)).astype(np.float32)
    x = x.astype(np.float64)
    for s in (1.0, 0.625, 2.0 ** -3):
        np.testing.assert_array_equal(ox.elem_codes(x, s, 1.0), brute_e2m1(x, s, 1.0))


def test_elem_zero_scale_and_sign(ox):
    assert ox.elem_code(0.3, 0.0, 1.0) == 0
    assert ox.elem_code(-0.3, 0.0, 1.0) == 8
    assert ox.elem_code(-0.0, 1.0, 1.0) == 8
    assert ox.elem_code(-1e-30, 1.0, 1.0) == 8
    assert ox.elem_code(100.0, 1.0, 1.0) == 7  # clip to 6
    assert ox.elem_code(-100.0, 1.0, 1.0) == 15


# ----------------------------------------------------------------------------- scales


def _f32_range(lo: float, hi: float, stride: int) -> np.ndarray:
    a = np.array([lo, hi], dtype=np.float32).view(np.uint32).astype(np.int64)
    return np.arange(a[0], a[1] + 1, stride, dtype=np.int64).astype(np.uint32).view(np.float32)


def test_e4m3_scale_vs_torch(ox):
    vals = np.array([ox.scale_value(b, "e4m3") for b in range(0x7F)])
    mids = 0.5 * (vals[:-1] + vals[1:])
    v = np.concatenate([_f32_range(2.0 ** -14, 464.0, 97), around(mids, 2048).astype(np.float32),
                        around(vals[1:], 64).astype(np.float32)])
    v = v[(v > 0) & (v <= 464.0)].astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = ox.scale_bytes(6.0 * v.astype(np.float64), 1.0, "e4m3")  # a = 6 v exactly: a/6 == v
    np.testing.assert_array_equal(got, ref)


def test_e4m3_scale_saturates(ox):
    # above the last midpoint torch produces NaN; the oracle saturates at 448 (0x7E)
    for v in (464.0001, 470.0, 1e4, 3e38):
        assert ox.scale_byte(6.0 * v, 1.0, "e4m3") == 0x7E
    # flush: v <= 2^-10 (half the smallest subnormal, the tie going to the even code 0)
    assert ox.scale_byte(6.0 * 2.0 ** -10, 1.0, "e4m3") == 0
    assert ox.scale_byte(np.nextafter(6.0 * 2.0 ** -10, 1.0), 1.0, "e4m3") == 1


def test_e8m0_scale_vs_torch(ox):
    vs = []
    for e in range(-133, 127):
        base = 2.0 ** e
        vs.append(np.array([base, 1.25 * base, 1.5 * base, 1.75 * base, 1.9999 * base],
                           dtype=np.float32))
        vs.append(around([1.5 * base], 8).astype(np.float32))
    v = np.concatenate(vs)
    v = v[(v > 0) & np.isfinite(v) & (v < 1.5 * 2.0 ** 127)].astype(np.float32)
    # torch rounds fp32-subnormal inputs on their bit pattern (1.25 * 2^-127 -> 2^-126), which
    # is not the nearest value; compare with torch on normal fp32 inputs only ...
    normal = v >= 2.0 ** -126
    ref = torch.from_numpy(v[normal]).to(torch.float8_e8m0fnu).view(torch.uint8).numpy()
    got = ox.scale_bytes(6.0 * v[normal].astype(np.float64), 1.0, "e8m0")
    np.testing.assert_array_equal(got, ref)
    # ... and below 2^-126 with the brute-force nearest power of two (ties up)
    sub = v[~normal].astype(np.float64)
    d0, d1 = np.abs(sub - 2.0 ** -127), np.abs(sub - 2.0 ** -126)
    np.testing.assert_array_equal(ox.scale_bytes(6.0 * sub, 1.0, "e8m0"),
                                  np.where(d1 <= d0, 1, 0).astype(np.uint8))
    # zero and the saturation end
    assert ox.scale_byte(0.0, 1.0, "e8m0") == 0
    assert ox.scale_byte(6.0 * 1.6 * 2.0 ** 127, 1.0, "e8m0") == 0xFE


def test_ue5m3_scale_brute_force(ox):
    vals = np.array([ox.scale_value(b, "ue5m3") for b in range(255)])
    mids = 0.5 * (vals[:-1] + vals[1:])
    rng = np.random.default_rng(3)
    v = np.concatenate([
        around(mids, 256), around(vals[1:], 16),
        np.exp(rng.uniform(np.log(2.0 ** -20), np.log(2.0 ** 18), 200_000)).astype(np.float32),
    ]).astype(np.float64)
    v = v[v > 0]
    got = ox.scale_bytes(6.0 * v, 1.0, "ue5m3")
    # brute force in chunks: nearest of all 255 values, ties to the even code
    for i0 in range(0, len(v), 20000):
        vv = v[i0:i0 + 20000, None]
        d = np.abs(vv - vals[None, :])
        best = d.min(axis=1, keepdims=True)
        ties = d == best
        even = ties & (np.arange(255)[None, :] % 2 == 0)
        idx = np.where(even.any(axis=1), even.argmax(axis=1), ties.argmax(axis=1))
        np.testing.assert_array_equal(got[i0:i0 + 20000], idx.astype(np.uint8))


@pytest.mark.parametrize("fmt", ["e4m3", "ue5m3", "e8m0"])
def test_scale_of_fl32_quotient_is_exact(ox, fmt):
    """Rounding fl32(a/6) onto the scale format gives the byte of the exact a/6, for fp32 a
    (bf16 absmax values are a subset).  Dense around every 6 x midpoint and sampled elsewhere."""
    vals = np.array([ox.scale_value(b, fmt) for b in range(0x7F if fmt == "e4m3" else 0xFF)])
    mids = 0.5 * (vals[:-1] + vals[1:])
    mids = mids[(6 * mids < 3e38) & (6 * mids > 1e-37)]
    a = np.concatenate([around(6.0 * mids, 512), _f32_range(1e-36, 3e38, 104729)]).astype(np.float32)
    q = (a / np.float32(6.0)).astype(np.float32)  # correctly rounded fp32 division
    exact = ox.scale_bytes(a.astype(np.float64), 1.0, fmt)
    via_q = ox.scale_bytes(6.0 * q.astype(np.float64), 1.0, fmt)
    np.testing.assert_array_equal(exact, via_q)


@pytest.mark.parametrize("fmt", ["e4m3", "ue5m3", "e8m0"])
def test_scale_of_f64_reciprocal_product_is_exact(ox, fmt):
    """Rounding fl32(fl64(a) * fl64(1/6)) onto the scale format also gives the byte of the
    exact a/6 (the product lands on a midpoint exactly when a/6 does, and otherwise stays far
    enough from it); the GPU scale path computes the quotient this way."""
    vals = np.array([ox.scale_value(b, fmt) for b in range(0x7F if fmt == "e4m3" else 0xFF)])
    mids = 0.5 * (vals[:-1] + vals[1:])
    mids = mids[(6 * mids < 3e38) & (6 * mids > 1e-37)]
    a = np.concatenate([around(6.0 * mids, 512), _f32_range(1e-36, 3e38, 104729)]).astype(np.float32)
    q = (a.astype(np.float64) * (1.0 / 6.0)).astype(np.float32)
    exact = ox.scale_bytes(a.astype(np.float64), 1.0, fmt)
    via_q = ox.scale_bytes(6.0 * q.astype(np.float64), 1.0, fmt)
    np.testing.assert_array_equal(exact, via_q)


def _f32_neighbours(v: float) -> np.ndarray:
    """The fp32 values adjacent to the real v: the largest fp32 below, the smallest above, and v
    itself when it is an fp32 value (v >= 0, v within the fp32 range)."""
    f = np.float32(v)
    lo = f if float(f) <= v else np.nextafter(f, np.float32(0))
    hi = f if float(f) >= v else np.nextafter(f, np.float32(np.inf))
    cand = [np.nextafter(lo, np.float32(0)), lo, hi, np.nextafter(hi, np.float32(np.inf))]
    return np.array(cand, dtype=np.float32)


@pytest.mark.parametrize("fmt", ["e4m3", "ue5m3", "e8m0"])
def test_scale_of_fl32_quotient_is_exact_for_every_fp32(ox, fmt):
    """Proof, for every positive finite fp32 a, that rounding fl32(a/6) onto the scale format
    gives the byte of the exact a/6.  Both maps a -> byte are non-decreasing step functions of
    a (fl32 division and nearest rounding are monotone).  The exact one steps only where a/6
    crosses a midpoint between neighbouring scale values; if the two maps agree on the fp32
    values on either side of every such step and at both ends of the fp32 range, then on each
    interval between steps the quotient map is squeezed between equal values, so they agree
    everywhere.  Checked: both neighbours (and one more on each side) of 6 x every midpoint
    inside the fp32 range, the smallest subnormal and the largest finite fp32."""
    vals = np.array([ox.scale_value(b, fmt) for b in range(0x7F if fmt == "e4m3" else 0xFF)])
    mids = 0.5 * (vals[:-1] + vals[1:])
    fmax = float(np.finfo(np.float32).max)
    pts = [np.array([2.0 ** -149, fmax], dtype=np.float32)]
    # the flush step of E4M3 / UE5M3 sits at half the smallest subnormal scale (included in mids
    # as the midpoint between 0 and it); E8M0 has no zero, its lowest step is between 2^-127 and
    # 2^-126
    for m in mids:
        if 2.0 ** -149 <= 6.0 * m <= fmax:
            pts.append(_f32_neighbours(6.0 * m))
    a = np.concatenate(pts)
    a = a[(a > 0) & np.isfinite(a)]
    q = (a / np.float32(6.0)).astype(np.float32)
    exact = ox.scale_bytes(a.astype(np.float64), 1.0, fmt)
    via_q = ox.scale_bytes(6.0 * q.astype(np.float64), 1.0, fmt)
    np.testing.assert_array_equal(exact, via_q)
    # and the exact map does step at each of those midpoints (the premise of the argument)
    inside = [m for m in mids if 2.0 ** -149 <= 6.0 * m <= fmax]
    assert len(inside) > 10
