"""Helpers for the GPU parity tests: host<->device conversion, edge-case inputs, tolerance."""
from __future__ import annotations

import numpy as np
import torch

import oracle

DEV = "cuda:0"


def bf16_dev(a: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bits (numpy) -> bf16 tensor on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)


def f32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 bits; fp32 -> float32; uint8 -> uint8."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bf16_bits(v) -> np.ndarray:
    """Nearest-even bf16 bits of float values (exact for values that are bf16)."""
    f = np.asarray(v, dtype=np.float32)
    return torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def edge_tensor(k: int = 512, seed: int = 1) -> np.ndarray:
    """bf16 rows (k elements each) that, for block 32, hit every finite scale byte of every
    format, every bf16 magnitude in [0, 6] under scale 1, exact ties t*s for every scale
    mantissa, zero / -0 / flush-boundary / saturating / subnormal blocks."""
    rng = np.random.default_rng(seed)
    blocks = []

    def block_with_max(a: float, rest: np.ndarray):
        b = np.empty(32, dtype=np.float32)
        b[0] = a
        b[1:] = rest
        blocks.append(b)

    # every finite positive scale byte: absmax = 6 s (exact in bf16 when in range)
    for fmt in ("e4m3", "ue5m3", "e8m0"):
        for byte in range(256):
            s = oracle.scale_value(byte, fmt)
            if not np.isfinite(s) or s <= 0 or 6 * s > 3.0e38 or 6 * s < 1e-38:
                continue
            a = 6.0 * s
            rest = (rng.uniform(-1, 1, 31) * a).astype(np.float32)
            block_with_max(a, rest)
    # all bf16 magnitudes in (0, 6], both signs, under an absmax of 6
    mags = np.arange(1, 0x40C1, dtype=np.uint32)  # bf16 bits 0x0001 .. 0x40C0 (6.0)
    vals = (mags << 16).view(np.float32)
    vals = np.concatenate([vals, -vals])
    for i in range(0, len(vals), 31):
        chunk = vals[i:i + 31]
        rest = np.zeros(31, dtype=np.float32)
        rest[:len(chunk)] = chunk
        block_with_max(6.0, rest)
    # exact ties and neighbours for every scale mantissa (E4M3/UE5M3) at a few exponents
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1, 1.5, 2, 3, 4])
    for mi in range(8):
        for e in (-9, -3, 0, 4):
            s = (1 + mi / 8) * 2.0 ** e
            t = (ties * s).astype(np.float32)
            tb = bf16_bits(t).astype(np.int32)
            nb = np.concatenate([tb, tb + 1, tb - 1]).astype(np.uint16)
            rest = (nb.astype(np.uint32) << 16).view(np.float32)
            rest = np.concatenate([rest, -rest[:2]])[:31]
            rest = np.pad(rest, (0, 31 - len(rest)))
            block_with_max(6.0 * s, rest)
    # signed zeros inside blocks with a non-zero scale (the sign bit must survive)
    for mi in range(8):
        rest = np.zeros(31, dtype=np.float32)
        rest[1::2] = -0.0
        rest[4] = -2.0 ** -133
        block_with_max(6.0 * (1 + mi / 8), rest)
    # special blocks
    z = np.zeros(31, dtype=np.float32)
    block_with_max(0.0, z)
    block_with_max(-0.0, -z)
    for a in (3 * 2.0 ** -9, np.nextafter(np.float32(3 * 2.0 ** -9), np.float32(1)),
              3 * 2.0 ** -17, 1e4, 448 * 6.0, 3e38, 1e-38, 2.0 ** -133, 9 * 2.0 ** -10):
        block_with_max(a, (rng.uniform(-1, 1, 31) * a).astype(np.float32))
    x = np.concatenate(blocks)
    bits = bf16_bits(x)
    pad = (-len(bits)) % k
    bits = np.concatenate([bits, bf16_bits(rng.standard_normal(pad).astype(np.float32))])
    return bits.reshape(-1, k)


def assert_gemm_close(y_gpu: np.ndarray, y_ref: np.ndarray, a_ref: np.ndarray, bf16_out: bool,
                      what: str):
    """|Y - Yref| <= 2e-5 * sum|x w|, plus half a bf16 ulp of Yref for bf16 output."""
    y = y_gpu.astype(np.float64)
    tol = 2e-5 * a_ref
    if bf16_out:
        mag = np.abs(y_ref)
        e = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
        tol = tol + np.where(mag > 0, 2.0 ** (e - 8), 2.0 ** -133)
    err = np.abs(y - y_ref)
    bad = err > tol
    if bad.any():
        i = np.argmax(err / np.maximum(tol, 1e-300))
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outputs out of tolerance; worst "
                             f"idx {np.unravel_index(i, y.shape)} got {y.flat[i]!r} ref "
                             f"{y_ref.flat[i]!r} tol {tol.flat[i]!r}")


# Tiled scale layout (include/mx.h, MX_LAYOUT_TILED), written out from its definition.
def tiled_positions(rows: int, k: int) -> np.ndarray:
    """Byte position of the scale of (r, b) for every row r and 32-element block b."""
    ks = -(-k // 256)
    r = np.arange(rows)[:, None]
    b = np.arange(k // 32)[None, :]
    t = r % 256
    return (2048 * ((r // 256) * ks + b // 8) + 1024 * (t // 128) + 32 * (t % 32)
            + 8 * ((t // 32) % 4) + b % 8)


def padding_positions(rows: int, k: int) -> np.ndarray:
    ks = -(-k // 256)
    nb = k // 32
    pads = []
    for b in range(nb, 8 * ks):
        r = np.arange(rows)
        t = r % 256
        pads.append(2048 * ((r // 256) * ks + b // 8) + 1024 * (t // 128) + 32 * (t % 32)
                    + 8 * ((t // 32) % 4) + b % 8)
    return np.concatenate(pads) if pads else np.zeros(0, dtype=np.int64)


def preshuffled_positions(rows: int, k: int) -> np.ndarray:
    """Byte offsets of the preshuffled scale layout (block 32) for a rows x k/32 row-major scale
    array: (r, b) -> 512 (R KC + C) + 8 u + t with R, t = divmod(r, 8), C, u = divmod(b, 64)."""
    nb = k // 32
    kc = (nb + 63) // 64
    r = np.arange(rows)[:, None]
    b = np.arange(nb)[None, :]
    return 512 * ((r // 8) * kc + b // 64) + 8 * (b % 64) + r % 8


def preshuffled_padding_positions(rows: int, k: int) -> np.ndarray:
    """Bytes of the last chunk past each row's last block (written as zero)."""
    nb = k // 32
    kc = (nb + 63) // 64
    pads = []
    for b in range(nb, 64 * kc):
        r = np.arange(rows)
        pads.append(512 * ((r // 8) * kc + b // 64) + 8 * (b % 64) + r % 8)
    return np.concatenate(pads) if pads else np.zeros(0, dtype=np.int64)
