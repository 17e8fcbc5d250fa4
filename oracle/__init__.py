"""CPU oracle for MX FP4 quantization and the FP4-weight matmul (ctypes over mxoracle.c).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It shares no code with the HIP library in
microscaling_fp4_weight_amd/, and the library never imports it.

Formats are named 'e4m3', 'ue5m3', 'e8m0'; element dtypes 'f32' (float32 arrays) and
'bf16' (uint16 arrays of bf16 bits).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxoracle.c")
_HDR = os.path.join(_HERE, "mxoracle.h")
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

FMT = {"e4m3": 0, "ue5m3": 1, "e8m0": 2}
DTYPE = {"f32": 0, "bf16": 1}
MODE = {"a16": 0, "a4": 1}


def build() -> str:
    """Compile mxoracle.c (single-threaded, -O2, IEEE, no contraction) into liboracle.so."""
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           _SRC, "-o", _SO + ".tmp", "-lm"]
    subprocess.check_call(cmd)
    os.replace(_SO + ".tmp", _SO)
    return _SO


def _load():
    global _lib
    if _lib is not None:
        return _lib
    newest = max(os.path.getmtime(_SRC), os.path.getmtime(_HDR))
    if not os.path.exists(_SO) or os.path.getmtime(_SO) < newest:
        build()
    lib = ctypes.CDLL(_SO)
    i32, i64, u32, f32, dbl, vp = (ctypes.c_int, ctypes.c_int64, ctypes.c_uint, ctypes.c_float,
                                   ctypes.c_double, ctypes.c_void_p)
    lib.ox_e2m1_value.argtypes = [u32]
    lib.ox_e2m1_value.restype = dbl
    lib.ox_scale_value.argtypes = [u32, i32]
    lib.ox_scale_value.restype = dbl
    lib.ox_scale_byte.argtypes = [dbl, dbl, i32]
    lib.ox_scale_byte.restype = u32
    lib.ox_elem_code.argtypes = [dbl, dbl, dbl]
    lib.ox_elem_code.restype = u32
    lib.ox_quantize.argtypes = [vp, i32, i64, i64, i64, i32, i32, f32, vp, vp]
    lib.ox_quantize.restype = i32
    lib.ox_dequantize.argtypes = [vp, vp, i64, i64, i32, i32, f32, vp, i32, i64]
    lib.ox_dequantize.restype = i32
    lib.ox_f32_to_bf16.argtypes = [f32]
    lib.ox_f32_to_bf16.restype = ctypes.c_uint16
    lib.ox_gemm.argtypes = [vp, i64, i64, i64, vp, vp, i64, i32, i32, f32, i32, vp, i64, vp, i64,
                            vp, vp]
    lib.ox_gemm.restype = i32
    lib.ox_mse_split.argtypes = [vp, i32, i64, i64, i64, i32, i32, f32, vp]
    lib.ox_mse_split.restype = i32
    lib.ox_scale_bytes.argtypes = [vp, i64, dbl, i32, vp]
    lib.ox_scale_bytes.restype = None
    lib.ox_elem_codes.argtypes = [vp, i64, dbl, dbl, vp]
    lib.ox_elem_codes.restype = None
    lib.ox_e4m3_value.argtypes = [u32]
    lib.ox_e4m3_value.restype = dbl
    lib.ox_scale_byte_fp8.argtypes = [dbl, dbl, i32]
    lib.ox_scale_byte_fp8.restype = u32
    lib.ox_elem_code_fp8.argtypes = [dbl, dbl, dbl]
    lib.ox_elem_code_fp8.restype = u32
    lib.ox_quantize_fp8.argtypes = [vp, i32, i64, i64, i64, i32, i32, f32, vp, vp]
    lib.ox_quantize_fp8.restype = i32
    lib.ox_dequantize_fp8.argtypes = [vp, vp, i64, i64, i32, i32, f32, vp, i32, i64]
    lib.ox_dequantize_fp8.restype = i32
    lib.ox_gemm_fp8.argtypes = [vp, i64, i64, i64, vp, vp, i64, i32, i32, f32, vp, i64, vp, i64, vp, vp]
    lib.ox_gemm_fp8.restype = i32
    lib.ox_scale_bytes_fp8.argtypes = [vp, i64, dbl, i32, vp]
    lib.ox_scale_bytes_fp8.restype = None
    lib.ox_elem_codes_fp8.argtypes = [vp, i64, dbl, dbl, vp]
    lib.ox_elem_codes_fp8.restype = None
    _lib = lib
    return lib


def scale_bytes(a: np.ndarray, g: float, fmt: str) -> np.ndarray:
    """Vector form of scale_byte over float64 absmax values."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.uint8)
    _load().ox_scale_bytes(a.ctypes.data, a.size, g, FMT[fmt], out.ctypes.data)
    return out


def elem_codes(x: np.ndarray, s: float, g: float = 1.0) -> np.ndarray:
    """Vector form of elem_code over float64 element values."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint8)
    _load().ox_elem_codes(x.ctypes.data, x.size, s, g, out.ctypes.data)
    return out


def _dtype_of(x: np.ndarray) -> str:
    if x.dtype == np.float32:
        return "f32"
    if x.dtype == np.uint16:
        return "bf16"
    raise TypeError(f"oracle input must be float32 or uint16 (bf16 bits), got {x.dtype}")


def e2m1_value(code: int) -> float:
    return _load().ox_e2m1_value(code)


def scale_value(byte: int, fmt: str) -> float:
    return _load().ox_scale_value(byte, FMT[fmt])


def scale_byte(a: float, g: float, fmt: str) -> int:
    return _load().ox_scale_byte(a, g, FMT[fmt])


def elem_code(x: float, s: float, g: float) -> int:
    return _load().ox_elem_code(x, s, g)


def f32_to_bf16(f: float) -> int:
    return _load().ox_f32_to_bf16(f)


def quantize(x: np.ndarray, block: int, fmt: str, g: float = 1.0):
    """x: rows x k float32 or bf16 bits -> (codes rows x k/2 uint8, scales rows x k/block uint8)."""
    x = np.ascontiguousarray(x)
    rows, k = x.shape
    codes = np.empty((rows, k // 2), dtype=np.uint8)
    scales = np.empty((rows, k // block), dtype=np.uint8)
    rc = _load().ox_quantize(x.ctypes.data, DTYPE[_dtype_of(x)], rows, k, k, block, FMT[fmt],
                             g, codes.ctypes.data, scales.ctypes.data)
    if rc != 0:
        raise ValueError("oracle quantize: bad arguments")
    return codes, scales


def dequantize(codes: np.ndarray, scales: np.ndarray, k: int, block: int, fmt: str,
               g: float = 1.0, out: str = "f32") -> np.ndarray:
    codes = np.ascontiguousarray(codes)
    scales = np.ascontiguousarray(scales)
    rows = codes.shape[0]
    y = np.empty((rows, k), dtype=np.float32 if out == "f32" else np.uint16)
    rc = _load().ox_dequantize(codes.ctypes.data, scales.ctypes.data, rows, k, block, FMT[fmt],
                               g, y.ctypes.data, DTYPE[out], k)
    if rc != 0:
        raise ValueError("oracle dequantize: bad arguments")
    return y


def gemm(x_bf16: np.ndarray, wcodes: np.ndarray, wscales: np.ndarray, block: int, fmt: str,
         g: float = 1.0, mode: str = "a16", mrows=None, ncols=None):
    """fp64 Y[i][j] = sum_k Xhat[mrows[i]][k] * What[ncols[j]][k] and A = sum_k |Xhat*What|.
    Returns (Y, A) as float64 arrays of shape (len(mrows), len(ncols))."""
    x = np.ascontiguousarray(x_bf16)
    assert x.dtype == np.uint16
    m, k = x.shape
    n = wcodes.shape[0]
    wc = np.ascontiguousarray(wcodes)
    ws = np.ascontiguousarray(wscales)
    mr = np.arange(m, dtype=np.int64) if mrows is None else np.asarray(mrows, dtype=np.int64)
    nc = np.arange(n, dtype=np.int64) if ncols is None else np.asarray(ncols, dtype=np.int64)
    mr = np.ascontiguousarray(mr)
    nc = np.ascontiguousarray(nc)
    y = np.empty((len(mr), len(nc)), dtype=np.float64)
    a = np.empty_like(y)
    rc = _load().ox_gemm(x.ctypes.data, m, k, k, wc.ctypes.data, ws.ctypes.data, n, block,
                         FMT[fmt], g, MODE[mode], mr.ctypes.data, len(mr), nc.ctypes.data,
                         len(nc), y.ctypes.data, a.ctypes.data)
    if rc != 0:
        raise ValueError("oracle gemm: bad arguments")
    return y, a


def mse_split(x: np.ndarray, block: int, fmt: str, g: float = 1.0) -> dict:
    x = np.ascontiguousarray(x)
    rows, k = x.shape
    out = np.zeros(7, dtype=np.float64)
    rc = _load().ox_mse_split(x.ctypes.data, DTYPE[_dtype_of(x)], rows, k, k, block, FMT[fmt], g,
                              out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle mse_split: bad arguments")
    return {"elem": out[0], "max": out[1], "zero": out[2], "total": out[3],
            "blocks": int(out[4]), "zero_blocks": int(out[5]), "max_not6": int(out[6])}


# ----------------------------------------------------------------------------------------
# Block-size policy (hotelren.com/news/2192771, article "量化技术演进与微缩量化原理",
# section 6 item 2: the block size follows the tensor's standard deviation; section 5.1 item
# 1: a block size per layer kind).
# ----------------------------------------------------------------------------------------

def tensor_stats(x: np.ndarray) -> dict:
    """Mean, standard deviation and max |x| of a whole tensor, in fp64, by the textbook two
    passes: mean = sum(x) / n, then std = sqrt(sum((x - mean)^2) / (n - 1)) (the sample
    standard deviation, n - 1 in the denominator; NaN for a single element)."""
    v = x.astype(np.float64) if x.dtype != np.uint16 else (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    v = v.ravel()
    n = v.size
    mean = float(np.sum(v)) / n
    m2 = float(np.sum((v - mean) ** 2))
    std = float(np.sqrt(m2 / (n - 1))) if n > 1 else float("nan")
    return {"mean": mean, "std": std, "absmax": float(np.max(np.abs(v))), "n": n}


def adaptive_block_size(sigma: float) -> int:
    """Section 6 item 2: sigma < 0.01 -> 128; sigma < 0.1 -> 64; otherwise 32."""
    if sigma < 0.01:
        return 128
    if sigma < 0.1:
        return 64
    return 32


LAYER_BLOCK = {"qkv": 64, "ffn_gate_up": 32, "output": 128}  # section 5.1 item 1


def layer_block_size(kind: str) -> int:
    """Section 5.1 item 1: Q/K/V projections 64, FFN gate/up 32, output projection 128."""
    return LAYER_BLOCK[kind]



# ----------------------------------------------------------------------------------------
# FP8 weight fallback (hotelren.com/news/2192771, article "量化技术演进与微缩量化原理",
# section 5.3 item 1: weights with sigma < 1e-4 are lost to FP4 and go to FP8 instead;
# section 6 item 1: key layers stay in FP8).  E4M3 elements (largest magnitude 448) in the
# same blocks under the same scale formats; the scale rule divides by 448 instead of 6.
# ----------------------------------------------------------------------------------------

def e4m3_value(code: int) -> float:
    return _load().ox_e4m3_value(code)


def scale_byte_fp8(a: float, g: float, fmt: str) -> int:
    return _load().ox_scale_byte_fp8(a, g, FMT[fmt])


def elem_code_fp8(x: float, s: float, g: float = 1.0) -> int:
    return _load().ox_elem_code_fp8(x, s, g)


def scale_bytes_fp8(a: np.ndarray, g: float, fmt: str) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float64)
    out = np.empty(a.size, dtype=np.uint8)
    _load().ox_scale_bytes_fp8(a.ctypes.data, a.size, g, FMT[fmt], out.ctypes.data)
    return out.reshape(a.shape)


def elem_codes_fp8(x: np.ndarray, s: float, g: float = 1.0) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.size, dtype=np.uint8)
    _load().ox_elem_codes_fp8(x.ctypes.data, x.size, s, g, out.ctypes.data)
    return out.reshape(x.shape)


def quantize_fp8(x: np.ndarray, block: int, fmt: str, g: float = 1.0):
    """x: rows x k float32 or bf16 bits -> (codes rows x k uint8, scales rows x k/block uint8)."""
    x = np.ascontiguousarray(x)
    rows, k = x.shape
    codes = np.empty((rows, k), dtype=np.uint8)
    scales = np.empty((rows, k // block), dtype=np.uint8)
    rc = _load().ox_quantize_fp8(x.ctypes.data, DTYPE[_dtype_of(x)], rows, k, k, block, FMT[fmt],
                                 g, codes.ctypes.data, scales.ctypes.data)
    if rc != 0:
        raise ValueError("oracle quantize_fp8: bad arguments")
    return codes, scales


def dequantize_fp8(codes: np.ndarray, scales: np.ndarray, block: int, fmt: str, g: float = 1.0,
                   out: str = "f32") -> np.ndarray:
    codes = np.ascontiguousarray(codes)
    scales = np.ascontiguousarray(scales)
    rows, k = codes.shape
    y = np.empty((rows, k), dtype=np.float32 if out == "f32" else np.uint16)
    rc = _load().ox_dequantize_fp8(codes.ctypes.data, scales.ctypes.data, rows, k, block, FMT[fmt],
                                   g, y.ctypes.data, DTYPE[out], k)
    if rc != 0:
        raise ValueError("oracle dequantize_fp8: bad arguments")
    return y


def gemm_fp8(x_bf16: np.ndarray, wcodes: np.ndarray, wscales: np.ndarray, block: int, fmt: str,
             g: float = 1.0, mrows=None, ncols=None):
    """Y = X . dequant(W8)^T in fp64 and A = sum |x w| (bf16 X), for the selected rows/columns."""
    x = np.ascontiguousarray(x_bf16)
    m, k = x.shape
    n = wcodes.shape[0]
    mr = np.arange(m, dtype=np.int64) if mrows is None else np.ascontiguousarray(mrows, dtype=np.int64)
    nc = np.arange(n, dtype=np.int64) if ncols is None else np.ascontiguousarray(ncols, dtype=np.int64)
    wc = np.ascontiguousarray(wcodes)
    ws = np.ascontiguousarray(wscales)
    y = np.empty((mr.size, nc.size), dtype=np.float64)
    a = np.empty_like(y)
    rc = _load().ox_gemm_fp8(x.ctypes.data, m, k, k, wc.ctypes.data, ws.ctypes.data, n, block, FMT[fmt],
                             g, mr.ctypes.data, mr.size, nc.ctypes.data, nc.size, y.ctypes.data, a.ctypes.data)
    if rc != 0:
        raise ValueError("oracle gemm_fp8: bad arguments")
    return y, a


def use_fp8(sigma: float) -> bool:
    """Section 5.3 item 1: a weight tensor with sigma < 1e-4 takes the FP8 fallback."""
    return sigma < 1e-4
