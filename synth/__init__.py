"""Seeded synthetic input tensors shared by the tests, the smoke check and the benchmark.

The generator (synth.c) is counter-based: element i of tensor (seed, stream) depends
only on (seed, stream, i), so any row range can be regenerated on its own and the
bytes do not depend on the thread count.  It contains no quantization arithmetic.

`recipe(name)` gives the tensors of each workload by name; the shapes, spreads and
outlier rates follow the workloads' descriptions (Llama-shaped weights, N(0, sigma^2)
entries, a Bernoulli fraction of entries multiplied by 20).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_SO = os.path.join(_HERE, "libsynth.so")
_lib = None


def build() -> str:
    """Compile synth.c into libsynth.so (always recompiles)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           _SRC, "-o", _SO + ".tmp", "-lm"]
    subprocess.check_call(cmd)
    os.replace(_SO + ".tmp", _SO)
    return _SO


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_SO)
    i64, u64, dbl, vp = ctypes.c_int64, ctypes.c_uint64, ctypes.c_double, ctypes.c_void_p
    lib.synth_normal_f32.argtypes = [vp, i64, i64, u64, u64, dbl, dbl, dbl]
    lib.synth_normal_bf16.argtypes = [vp, i64, i64, u64, u64, dbl, dbl, dbl]
    lib.synth_banded_bf16.argtypes = [vp, i64, i64, i64, i64, u64, u64, i64, i64, i64, dbl, dbl,
                                      dbl, dbl]
    for f in (lib.synth_normal_f32, lib.synth_normal_bf16, lib.synth_banded_bf16):
        f.restype = None
    _lib = lib
    return lib


def stream_id(name: str) -> int:
    """64-bit FNV-1a hash of a tensor name: the generator's stream number."""
    h = 0xCBF29CE484222325
    for b in name.encode():
        h ^= b
        h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def normal(shape, dtype: str, name: str, sigma: float, p_out: float = 0.0, mult: float = 20.0,
           seed: int = 0, row0: int = 0, nrows: int | None = None) -> np.ndarray:
    """Rows [row0, row0+nrows) of a 2-D tensor of N(0, sigma^2) entries; a Bernoulli(p_out)
    fraction is multiplied by `mult`.  dtype 'f32' -> float32, 'bf16' -> uint16 bits."""
    rows, k = int(shape[0]), int(shape[1])
    nrows = rows - row0 if nrows is None else nrows
    assert 0 <= row0 and row0 + nrows <= rows
    lib = _load()
    count = nrows * k
    if dtype == "f32":
        out = np.empty((nrows, k), dtype=np.float32)
        lib.synth_normal_f32(out.ctypes.data, row0 * k, count, seed, stream_id(name), sigma,
                             p_out, mult)
    elif dtype == "bf16":
        out = np.empty((nrows, k), dtype=np.uint16)
        lib.synth_normal_bf16(out.ctypes.data, row0 * k, count, seed, stream_id(name), sigma,
                              p_out, mult)
    else:
        raise ValueError(dtype)
    return out


def banded_bf16(shape, name: str, bands: int, period: int, phase: int, sigma: float,
                sigma_alt: float, p_out: float = 0.0, mult: float = 20.0, seed: int = 0,
                row0: int = 0, nrows: int | None = None) -> np.ndarray:
    """bf16 matrix whose rows form `bands` contiguous bands; bands with index % period == phase
    use sigma_alt, the others sigma."""
    rows, k = int(shape[0]), int(shape[1])
    nrows = rows - row0 if nrows is None else nrows
    assert rows % bands == 0 and 0 <= row0 and row0 + nrows <= rows
    lib = _load()
    out = np.empty((nrows, k), dtype=np.uint16)
    lib.synth_banded_bf16(out.ctypes.data, row0, nrows, rows, k, seed, stream_id(name), bands,
                          period, phase, sigma, sigma_alt, p_out, mult)
    return out


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bits to float32."""
    return (a.astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------------------
# Workloads.  Each entry: a function (rows0, nrows) -> array for every tensor it uses.
# ----------------------------------------------------------------------------------------

C2_SIGMAS = (0.005, 0.02, 0.1)
C2_BLOCKS = (4, 8, 16, 32, 64, 128, 256)
C2_FORMATS = ("e4m3", "ue5m3", "e8m0")


def c1_weight(row0=0, nrows=None):
    """256 x 256 fp32 weight ~ N(0, 0.02^2), 1% of entries x20, seed 0."""
    return normal((256, 256), "f32", "c1.w", 0.02, 0.01, 20.0, row0=row0, nrows=nrows)


def c1_x():
    """1 x 256 bf16 activation ~ N(0, 1)."""
    return normal((1, 256), "bf16", "c1.x", 1.0)


def c2_weight(sigma: float, row0=0, nrows=None):
    """Llama-7B FFN-shaped bf16 weight 4096 x 11008 ~ N(0, sigma^2), 0.1% of entries x20."""
    return normal((4096, 11008), "bf16", f"c2.w.{sigma}", sigma, 0.001, 20.0, row0=row0,
                  nrows=nrows)


def c3_x(m: int):
    """Decode activations M x 4096 bf16 ~ N(0, 1)."""
    return normal((m, 4096), "bf16", f"c3.x.{m}", 1.0)


def c3_weight(n: int, copy: int = 0, row0=0, nrows=None):
    """Decode weight N x 4096 bf16 ~ N(0, 0.02^2); `copy` selects one of several distinct
    matrices of the same shape."""
    return normal((n, 4096), "bf16", f"c3.w.{n}.{copy}", 0.02, row0=row0, nrows=nrows)


def c4_x(row0=0, nrows=None):
    """Prefill activations 2048 x 8192 bf16 ~ N(0, 1)."""
    return normal((2048, 8192), "bf16", "c4.x", 1.0, row0=row0, nrows=nrows)


def c4_weight(row0=0, nrows=None):
    """70B FFN weight 28672 x 8192 bf16 ~ N(0, 0.015^2), 0.1% of entries x20."""
    return normal((28672, 8192), "bf16", "c4.w", 0.015, 0.001, 20.0, row0=row0, nrows=nrows)


def c5_x(m: int, row0=0, nrows=None):
    """405B FFN activations M x 16384 bf16 ~ N(0, 1)."""
    return normal((m, 16384), "bf16", f"c5.x.{m}", 1.0, row0=row0, nrows=nrows)


def c5_weight(row0=0, nrows=None):
    """405B FFN weight 53248 x 16384 bf16: 16 contiguous row bands of 3328 rows; bands with
    index 3 mod 4 at sigma 0.02 (the narrow layers mixed in), the rest at 0.01."""
    return banded_bf16((53248, 16384), "c5.w", 16, 4, 3, 0.01, 0.02, row0=row0, nrows=nrows)


def absmax_bf16(a: np.ndarray) -> float:
    """max |x| of a bf16-bits array (the largest magnitude bit pattern)."""
    m = np.uint16(np.max(a & np.uint16(0x7FFF)))
    return float(bf16_to_f32(np.array([m], dtype=np.uint16))[0])


def c5_tensor_scale(w: np.ndarray) -> float:
    """Per-tensor scale of the 405B FFN weight: g = fl32(max|W| / (6 * 114688)), which puts the
    largest block's UE5M3 scale at the top of the format's range."""
    return float(np.float32(absmax_bf16(w) / (6.0 * 114688.0)))
