"""MX FP4 block quantization and FP4-weight GEMV/GEMM on AMD MI355X (gfx950).

A thin ctypes binding over libmx.so, whose C ABI is declared in include/mx.h.  Every
function here only marshals torch tensors (device memory) and the current HIP stream into
that ABI: all arithmetic runs in the library's HIP kernels.  There is no CPU fallback;
importing this package without a built libmx.so raises.

    import microscaling_fp4_weight_amd as mx
    codes, scales = mx.mx_quantize(w, block=32, fmt="e8m0")          # w: (n, k) bf16 / f32 on GPU
    w_hat = mx.mx_dequantize(codes, scales, k, 32, "e8m0", out_dtype=torch.bfloat16)
    y = mx.mx_gemm(x, codes, scales, block=32, fmt="e8m0", mode="a4")  # y = x . dequant(w)^T
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["mx_quantize", "mx_dequantize", "mx_gemm", "mx_gemm_workspace_size", "mx_scale_bytes",
           "mx_quant_error", "mx_quant_error_workspace_size",
           "mx_status_string", "MXError", "lib", "FMT", "MODE", "DTYPE", "LAYOUT", "STATUS"]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmx.so")

FMT = {"e4m3": 0, "ue5m3": 1, "e8m0": 2}
DTYPE = {"f32": 0, "bf16": 1}
MODE = {"a16": 0, "a4": 1}
LAYOUT = {"rowmajor": 0, "tiled": 1, "preshuffled": 2}
STATUS = {0: "MX_OK", -1: "MX_ERR_INVALID_ARG", -2: "MX_ERR_UNSUPPORTED", -3: "MX_ERR_ALIGNMENT",
          -4: "MX_ERR_HIP", -5: "MX_ERR_TOO_LARGE"}
GEMM_STATIC_SCRATCH_BYTES = 32 << 20  # MX_GEMM_STATIC_SCRATCH_BYTES in include/mx.h

_lib = None


class MXError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {STATUS.get(status, status)} ({mx_status_string(status)})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libmx.so with argument types set (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m microscaling_fp4_weight_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    i32, i64, f32, vp, sz = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
    L.mx_quantize.argtypes = [vp, i32, i64, i64, i64, i32, i32, f32, i32, vp, vp, vp]
    L.mx_quantize.restype = i32
    L.mx_dequantize.argtypes = [vp, vp, i64, i64, i32, i32, f32, i32, vp, i32, i64, vp]
    L.mx_dequantize.restype = i32
    L.mx_scale_bytes.argtypes = [i64, i64, i32, i32]
    L.mx_scale_bytes.restype = sz
    L.mx_quant_error_workspace_size.argtypes = [i64, i64, i32]
    L.mx_quant_error_workspace_size.restype = sz
    L.mx_quant_error.argtypes = [vp, i32, i64, i64, i64, i32, i32, f32, vp, i64, vp, vp, sz, vp]
    L.mx_quant_error.restype = i32
    L.mx_tensor_stats_workspace_size.argtypes = [i64, i64]
    L.mx_tensor_stats_workspace_size.restype = sz
    L.mx_tensor_stats.argtypes = [vp, i32, i64, i64, i64, vp, vp, sz, vp]
    L.mx_tensor_stats.restype = i32
    L.mx_adaptive_block_size.argtypes = [ctypes.c_double]
    L.mx_adaptive_block_size.restype = i32
    L.mx_layer_block_size.argtypes = [i32]
    L.mx_layer_block_size.restype = i32
    L.mx_quantize_fp8.argtypes = [vp, i32, i64, i64, i64, i32, i32, f32, vp, vp, vp]
    L.mx_quantize_fp8.restype = i32
    L.mx_dequantize_fp8.argtypes = [vp, vp, i64, i64, i32, i32, f32, vp, i32, i64, vp]
    L.mx_dequantize_fp8.restype = i32
    L.mx_gemm_fp8.argtypes = [vp, i64, i64, i64, i64, vp, vp, i32, i32, f32, vp, i32, i64, vp]
    L.mx_gemm_fp8.restype = i32
    L.mx_use_fp8.argtypes = [ctypes.c_double]
    L.mx_use_fp8.restype = i32
    L.mx_gemm_workspace_size.argtypes = [i64, i64, i64, i32, i32]
    L.mx_gemm_workspace_size.restype = sz
    L.mx_gemm.argtypes = [vp, i64, i64, i64, i64, vp, vp, i32, i32, f32, i32, i32, vp, i32, i64, vp,
                          sz, vp]
    L.mx_gemm.restype = i32
    L.mx_gemm_static.argtypes = [vp, i64, i64, i64, i64, vp, vp, i32, i32, f32, i32, i32, vp, i32, i64, vp]
    L.mx_gemm_static.restype = i32
    L.mx_status_string.argtypes = [i32]
    L.mx_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def mx_status_string(status: int) -> str:
    return lib().mx_status_string(status).decode()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _check(status: int, where: str):
    if status != 0:
        raise MXError(status, where)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return DTYPE["bf16"]
    if dt == torch.float32:
        return DTYPE["f32"]
    raise TypeError(f"unsupported dtype {dt}")


def _rows_ld(t: torch.Tensor, name: str):
    if t.dim() != 2 or (t.size(1) > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be a 2-D tensor with unit stride along its last dimension")
    return t.size(0), t.size(1), t.stride(0) if t.size(0) > 1 else t.size(1)


# Argument checks made before anything reaches the library: the C ABI trusts its pointers
# and sizes, so a tensor of the wrong dtype, shape or device would be read or written out of
# bounds on the GPU.  Dtypes and sizes are checked first, the device last.

def _need_dtype(t: torch.Tensor, name: str, dtypes):
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must be of dtype {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")


def _need_bytes(t: torch.Tensor, name: str, nbytes: int):
    """A contiguous uint8 buffer of at least nbytes bytes."""
    _need_dtype(t, name, (torch.uint8,))
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < nbytes:
        raise ValueError(f"{name} holds {t.numel()} bytes, {nbytes} needed")


def _need_shape(t: torch.Tensor, name: str, shape):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _need_gpu(**tensors):
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (device {t.device})")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")


def mx_quantize(x: torch.Tensor, block: int, fmt: str, tensor_scale: float = 1.0,
                layout: str = "rowmajor", codes: torch.Tensor | None = None,
                scales: torch.Tensor | None = None, stream=None):
    """MX-quantize a 2-D bf16/fp32 GPU tensor (rows x k) along k.
    Returns (codes uint8 rows x k/2, scales uint8: rows x k/block for layout "rowmajor", a
    flat buffer of mx_scale_bytes(...) bytes for layouts "tiled" and "preshuffled")."""
    rows, k, ld = _rows_ld(x, "x")
    _need_dtype(x, "x", (torch.bfloat16, torch.float32))
    if codes is None:
        codes = torch.empty((rows, k // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        if layout == "rowmajor":
            scales = torch.empty((rows, k // max(block, 1)), dtype=torch.uint8, device=x.device)
        else:
            scales = torch.empty(max(mx_scale_bytes(rows, k, block, layout), 1), dtype=torch.uint8,
                                 device=x.device)
    _need_bytes(codes, "codes", rows * (k // 2))
    _need_bytes(scales, "scales", mx_scale_bytes(rows, k, block, layout))
    _need_gpu(x=x, codes=codes, scales=scales)
    st = lib().mx_quantize(_ptr(x), _dtype_code(x.dtype), rows, k, ld, block, FMT[fmt],
                           tensor_scale, LAYOUT[layout], _ptr(codes), _ptr(scales), _stream(stream))
    _check(st, "mx_quantize")
    return codes, scales


def mx_dequantize(codes: torch.Tensor, scales: torch.Tensor, k: int, block: int, fmt: str,
                  tensor_scale: float = 1.0, out_dtype: torch.dtype = torch.bfloat16,
                  layout: str = "rowmajor", y: torch.Tensor | None = None, stream=None):
    """y = e(code) * s * g as a rows x k tensor of out_dtype (bf16 or fp32)."""
    if codes.dim() != 2:
        raise ValueError("codes must be a 2-D tensor (rows x k/2)")
    rows = codes.size(0)
    _need_shape(codes, "codes", (rows, k // 2))
    _need_bytes(codes, "codes", rows * (k // 2))
    _need_bytes(scales, "scales", mx_scale_bytes(rows, k, block, layout))
    if y is None:
        y = torch.empty((rows, k), dtype=out_dtype, device=codes.device)
    _need_dtype(y, "y", (torch.bfloat16, torch.float32))
    _need_shape(y, "y", (rows, k))
    _, _, ld = _rows_ld(y, "y")
    _need_gpu(codes=codes, scales=scales, y=y)
    st = lib().mx_dequantize(_ptr(codes), _ptr(scales), rows, k, block, FMT[fmt], tensor_scale,
                             LAYOUT[layout], _ptr(y), _dtype_code(y.dtype), ld, _stream(stream))
    _check(st, "mx_dequantize")
    return y


def mx_scale_bytes(rows: int, k: int, block: int, layout: str = "rowmajor") -> int:
    return int(lib().mx_scale_bytes(rows, k, block, LAYOUT[layout]))


def mx_quant_error_workspace_size(rows: int, k: int, block: int) -> int:
    return int(lib().mx_quant_error_workspace_size(rows, k, block))


def mx_quant_error(x: torch.Tensor, block: int, fmt: str, tensor_scale: float = 1.0,
                   x_hat: torch.Tensor | None = None, out: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Error split of MX-quantizing x (rows x k, bf16/fp32 on the GPU), computed on the device.
    Returns a float64 device tensor of 7 values: MSE_elem, MSE_max, MSE_zero, MSE_total,
    blocks, flushed blocks, non-flushed blocks whose maximum is not coded +-6.  When x_hat
    (same shape and dtype as x) is given, the dequantized tensor is written into it."""
    rows, k, ld = _rows_ld(x, "x")
    _need_dtype(x, "x", (torch.bfloat16, torch.float32))
    ldh = 0
    if x_hat is not None:
        if x_hat.dtype != x.dtype or tuple(x_hat.shape) != tuple(x.shape):
            raise ValueError("x_hat must have the shape and dtype of x")
        _, _, ldh = _rows_ld(x_hat, "x_hat")
    if out is None:
        out = torch.zeros(8, dtype=torch.float64, device=x.device)  # 7 used; 16-byte aligned
    _need_dtype(out, "out", (torch.float64,))
    if not out.is_contiguous() or out.numel() < 7:
        raise ValueError("out must be a contiguous float64 tensor of at least 7 elements")
    need = mx_quant_error_workspace_size(rows, k, block)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _need_bytes(workspace, "workspace", need)
    _need_gpu(x=x, x_hat=x_hat, out=out, workspace=workspace)
    st = lib().mx_quant_error(_ptr(x), _dtype_code(x.dtype), rows, k, ld, block, FMT[fmt], tensor_scale,
                              _ptr(x_hat), ldh, _ptr(out), _ptr(workspace), workspace.numel(),
                              _stream(stream))
    _check(st, "mx_quant_error")
    return out[:7]


def mx_tensor_stats_workspace_size(rows: int, k: int) -> int:
    return int(lib().mx_tensor_stats_workspace_size(rows, k))


def mx_tensor_stats(x: torch.Tensor, out: torch.Tensor | None = None,
                    workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Mean, sample standard deviation and max |x| of a rows x k bf16/fp32 GPU tensor, computed
    on the device; returns a float64 device tensor of 3 values."""
    rows, k, ld = _rows_ld(x, "x")
    _need_dtype(x, "x", (torch.bfloat16, torch.float32))
    if out is None:
        out = torch.zeros(4, dtype=torch.float64, device=x.device)  # 3 used; 16-byte aligned
    _need_dtype(out, "out", (torch.float64,))
    if not out.is_contiguous() or out.numel() < 3:
        raise ValueError("out must be a contiguous float64 tensor of at least 3 elements")
    need = mx_tensor_stats_workspace_size(rows, k)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    _need_bytes(workspace, "workspace", need)
    _need_gpu(x=x, out=out, workspace=workspace)
    st = lib().mx_tensor_stats(_ptr(x), _dtype_code(x.dtype), rows, k, ld, _ptr(out), _ptr(workspace),
                               workspace.numel(), _stream(stream))
    _check(st, "mx_tensor_stats")
    return out[:3]


LAYER_KIND = {"qkv": 0, "ffn_gate_up": 1, "output": 2}


def mx_adaptive_block_size(sigma: float) -> int:
    return int(lib().mx_adaptive_block_size(sigma))


def mx_layer_block_size(kind: str) -> int:
    return int(lib().mx_layer_block_size(LAYER_KIND[kind]))


def mx_quantize_fp8(x: torch.Tensor, block: int, fmt: str, tensor_scale: float = 1.0,
                    codes: torch.Tensor | None = None, scales: torch.Tensor | None = None, stream=None):
    """FP8 (E4M3 element) MX quantization of x (rows x k, bf16/fp32 on the GPU) -> (codes rows x k
    uint8, scales rows x k/block uint8)."""
    rows, k, ld = _rows_ld(x, "x")
    _need_dtype(x, "x", (torch.bfloat16, torch.float32))
    if codes is None:
        codes = torch.empty((rows, k), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((rows, k // block if block else 0), dtype=torch.uint8, device=x.device)
    _need_bytes(codes, "codes", rows * k)
    _need_bytes(scales, "scales", mx_scale_bytes(rows, k, block))
    _need_gpu(x=x, codes=codes, scales=scales)
    st = lib().mx_quantize_fp8(_ptr(x), _dtype_code(x.dtype), rows, k, ld, block, FMT[fmt], tensor_scale,
                               _ptr(codes), _ptr(scales), _stream(stream))
    _check(st, "mx_quantize_fp8")
    return codes, scales


def mx_dequantize_fp8(codes: torch.Tensor, scales: torch.Tensor, block: int, fmt: str,
                      tensor_scale: float = 1.0, out_dtype: torch.dtype = torch.float32,
                      y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    if codes.dim() != 2:
        raise ValueError("codes must be a 2-D tensor (rows x k)")
    rows, k = codes.shape
    _need_bytes(codes, "codes", rows * k)
    _need_bytes(scales, "scales", mx_scale_bytes(rows, k, block))
    if y is None:
        y = torch.empty((rows, k), dtype=out_dtype, device=codes.device)
    _need_dtype(y, "y", (torch.bfloat16, torch.float32))
    _need_shape(y, "y", (rows, k))
    _, _, ldy = _rows_ld(y, "y")
    _need_gpu(codes=codes, scales=scales, y=y)
    st = lib().mx_dequantize_fp8(_ptr(codes), _ptr(scales), rows, k, block, FMT[fmt], tensor_scale, _ptr(y),
                                 _dtype_code(y.dtype), ldy, _stream(stream))
    _check(st, "mx_dequantize_fp8")
    return y


def mx_gemm_fp8(x: torch.Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor, block: int, fmt: str,
                tensor_scale: float = 1.0, out_dtype: torch.dtype = torch.bfloat16,
                y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Y = X . dequant(W8)^T; x: m x k bf16; w_codes: n x k; w_scales: n x k/block."""
    m, k, ldx = _rows_ld(x, "x")
    _need_dtype(x, "x", (torch.bfloat16,))
    if w_codes.dim() != 2 or w_codes.size(1) != k:
        raise ValueError(f"w_codes must be a 2-D tensor (n x {k})")
    n = w_codes.size(0)
    _need_bytes(w_codes, "w_codes", n * k)
    _need_bytes(w_scales, "w_scales", mx_scale_bytes(n, k, block))
    if y is None:
        y = torch.empty((m, n), dtype=out_dtype, device=x.device)
    _need_dtype(y, "y", (torch.bfloat16, torch.float32))
    _need_shape(y, "y", (m, n))
    _, _, ldy = _rows_ld(y, "y")
    _need_gpu(x=x, w_codes=w_codes, w_scales=w_scales, y=y)
    st = lib().mx_gemm_fp8(_ptr(x), m, n, k, ldx, _ptr(w_codes), _ptr(w_scales), block, FMT[fmt], tensor_scale,
                           _ptr(y), _dtype_code(y.dtype), ldy, _stream(stream))
    _check(st, "mx_gemm_fp8")
    return y


def mx_use_fp8(sigma: float) -> bool:
    return bool(lib().mx_use_fp8(sigma))


def mx_gemm_workspace_size(m: int, n: int, k: int, block: int, mode: str) -> int:
    return int(lib().mx_gemm_workspace_size(m, n, k, block, MODE[mode]))


def mx_gemm(x: torch.Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor, block: int, fmt: str,
            tensor_scale: float = 1.0, mode: str = "a16", out_dtype: torch.dtype = torch.bfloat16,
            layout: str = "rowmajor", y: torch.Tensor | None = None,
            workspace: torch.Tensor | None = None, stream=None):
    """Y = X . dequant(Wq)^T.  x: m x k bf16; w_codes: n x k/2; w_scales: n x k/block."""
    m, k, ldx = _rows_ld(x, "x")
    _need_dtype(x, "x", (torch.bfloat16,))
    if w_codes.dim() != 2 or w_codes.size(1) != k // 2:
        raise ValueError(f"w_codes must be a 2-D tensor (n x {k // 2})")
    n = w_codes.size(0)
    _need_bytes(w_codes, "w_codes", n * (k // 2))
    _need_bytes(w_scales, "w_scales", mx_scale_bytes(n, k, block, layout))
    if y is None:
        y = torch.empty((m, n), dtype=out_dtype, device=x.device)
    _need_dtype(y, "y", (torch.bfloat16, torch.float32))
    _need_shape(y, "y", (m, n))
    _, _, ldy = _rows_ld(y, "y")
    need = mx_gemm_workspace_size(m, n, k, block, mode)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if workspace is not None:
        _need_bytes(workspace, "workspace", need)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _need_gpu(x=x, w_codes=w_codes, w_scales=w_scales, y=y, workspace=workspace)
    st = lib().mx_gemm(_ptr(x), m, n, k, ldx, _ptr(w_codes), _ptr(w_scales), block, FMT[fmt],
                       tensor_scale, LAYOUT[layout], MODE[mode], _ptr(y), _dtype_code(y.dtype), ldy,
                       _ptr(workspace), wbytes, _stream(stream))
    _check(st, "mx_gemm")
    return y


def mx_gemm_static(x: torch.Tensor, w_codes: torch.Tensor, w_scales: torch.Tensor, block: int, fmt: str,
                   tensor_scale: float = 1.0, mode: str = "a16", out_dtype: torch.dtype = torch.bfloat16,
                   layout: str = "rowmajor", y: torch.Tensor | None = None, stream=None):
    """mx_gemm with the W4A4 workspace in the library's static device buffer (no allocation
    by the call; y must be given to keep the call allocation-free).  Calls that may overlap on
    one GPU race on that buffer."""
    m, k, ldx = _rows_ld(x, "x")
    _need_dtype(x, "x", (torch.bfloat16,))
    if w_codes.dim() != 2 or w_codes.size(1) != k // 2:
        raise ValueError(f"w_codes must be a 2-D tensor (n x {k // 2})")
    n = w_codes.size(0)
    _need_bytes(w_codes, "w_codes", n * (k // 2))
    _need_bytes(w_scales, "w_scales", mx_scale_bytes(n, k, block, layout))
    if y is None:
        y = torch.empty((m, n), dtype=out_dtype, device=x.device)
    _need_dtype(y, "y", (torch.bfloat16, torch.float32))
    _need_shape(y, "y", (m, n))
    _, _, ldy = _rows_ld(y, "y")
    _need_gpu(x=x, w_codes=w_codes, w_scales=w_scales, y=y)
    st = lib().mx_gemm_static(_ptr(x), m, n, k, ldx, _ptr(w_codes), _ptr(w_scales), block, FMT[fmt],
                              tensor_scale, LAYOUT[layout], MODE[mode], _ptr(y), _dtype_code(y.dtype), ldy,
                              _stream(stream))
    _check(st, "mx_gemm_static")
    return y
