"""The Python binding's argument checks (CPU only): tensors of the wrong dtype, shape, size,
layout in memory or device are rejected before any entry point that launches work is called.
The C ABI trusts its pointers and sizes, so these checks are what keeps a wrong tensor from
becoming an out-of-bounds access on the GPU."""
import pytest
import torch

import microscaling_fp4_weight_amd as mx

COMPUTE = {"mx_quantize", "mx_dequantize", "mx_gemm", "mx_quant_error", "mx_tensor_stats",
           "mx_quantize_fp8", "mx_dequantize_fp8", "mx_gemm_fp8"}


class _NoLaunch:
    """Forwards host-only functions of libmx (sizes, status strings); fails on compute ones."""

    def __init__(self, real):
        self._real = real

    def __getattr__(self, name):
        if name in COMPUTE:
            raise AssertionError(f"{name} reached the library")
        return getattr(self._real, name)


@pytest.fixture(autouse=True)
def no_launch(monkeypatch):
    real = mx.lib()
    monkeypatch.setattr(mx, "_lib", _NoLaunch(real))
    yield


bf, f32, u8 = torch.bfloat16, torch.float32, torch.uint8
M, N, K = 4, 64, 256


def _w():
    return torch.zeros((N, K // 2), dtype=u8), torch.zeros((N, K // 32), dtype=u8)


def test_gemm_rejects_fp32_activations():
    c, s = _w()
    with pytest.raises(TypeError):
        mx.mx_gemm(torch.zeros((M, K), dtype=f32), c, s, 32, "e8m0")


def test_gemm_rejects_wrong_code_shape_and_dtype():
    c, s = _w()
    x = torch.zeros((M, K), dtype=bf)
    with pytest.raises(ValueError):
        mx.mx_gemm(x, torch.zeros((N, K), dtype=u8), s, 32, "e8m0")
    with pytest.raises(TypeError):
        mx.mx_gemm(x, c.to(torch.int16), s, 32, "e8m0")
    with pytest.raises(ValueError):
        mx.mx_gemm(x, torch.zeros((N, K), dtype=u8)[:, ::2], s, 32, "e8m0")  # not contiguous


def test_gemm_rejects_short_scales_and_wrong_y():
    c, s = _w()
    x = torch.zeros((M, K), dtype=bf)
    with pytest.raises(ValueError):
        mx.mx_gemm(x, c, s[:-1], 32, "e8m0")
    with pytest.raises(ValueError):
        mx.mx_gemm(x, c, s, 16, "e8m0")  # block 16 needs twice the scale bytes
    with pytest.raises(ValueError):
        mx.mx_gemm(x, c, s, 32, "e8m0", y=torch.zeros((M, N - 1), dtype=bf))
    with pytest.raises(TypeError):
        mx.mx_gemm(x, c, s, 32, "e8m0", y=torch.zeros((M, N), dtype=torch.float16))


def test_gemm_rejects_short_workspace():
    c, s = _w()
    x = torch.zeros((M, K), dtype=bf)
    need = mx.mx_gemm_workspace_size(M, N, K, 32, "a4")
    with pytest.raises(ValueError):
        mx.mx_gemm(x, c, s, 32, "e8m0", mode="a4", workspace=torch.zeros(need - 1, dtype=u8))


def test_gemm_rejects_host_tensors():
    c, s = _w()
    with pytest.raises(ValueError, match="GPU tensor"):
        mx.mx_gemm(torch.zeros((M, K), dtype=bf), c, s, 32, "e8m0")


def test_quantize_checks():
    x = torch.zeros((M, K), dtype=bf)
    with pytest.raises(TypeError):
        mx.mx_quantize(x.to(torch.float16), 32, "e8m0")
    with pytest.raises(ValueError):
        mx.mx_quantize(x, 32, "e8m0", codes=torch.zeros((M, K // 2 - 1), dtype=u8))
    with pytest.raises(ValueError):
        mx.mx_quantize(x, 32, "e8m0", scales=torch.zeros((M, K // 32 - 1), dtype=u8))
    with pytest.raises(ValueError):
        mx.mx_quantize(x, 32, "e8m0", layout="preshuffled", scales=torch.zeros(511, dtype=u8))
    with pytest.raises(ValueError, match="GPU tensor"):
        mx.mx_quantize(x, 32, "e8m0")


def test_dequantize_checks():
    c = torch.zeros((M, K // 2), dtype=u8)
    s = torch.zeros((M, K // 32), dtype=u8)
    with pytest.raises(ValueError):
        mx.mx_dequantize(c, s, K + 2, 32, "e8m0")  # codes do not hold k / 2 bytes per row
    with pytest.raises(ValueError):
        mx.mx_dequantize(c, s[:, :-1], K, 32, "e8m0")
    with pytest.raises(ValueError):
        mx.mx_dequantize(c, s, K, 32, "e8m0", y=torch.zeros((M, K - 2), dtype=bf))
    with pytest.raises(ValueError, match="GPU tensor"):
        mx.mx_dequantize(c, s, K, 32, "e8m0")


def test_error_split_and_stats_checks():
    x = torch.zeros((M, K), dtype=bf)
    with pytest.raises(TypeError):
        mx.mx_quant_error(x, 32, "e8m0", out=torch.zeros(8, dtype=f32))
    with pytest.raises(ValueError):
        mx.mx_quant_error(x, 32, "e8m0", workspace=torch.zeros(1, dtype=u8))
    with pytest.raises(ValueError):
        mx.mx_tensor_stats(x, out=torch.zeros(2, dtype=torch.float64))
    with pytest.raises(ValueError, match="GPU tensor"):
        mx.mx_tensor_stats(x)


def test_fp8_checks():
    x = torch.zeros((M, K), dtype=bf)
    c8 = torch.zeros((N, K), dtype=u8)
    s8 = torch.zeros((N, K // 32), dtype=u8)
    with pytest.raises(TypeError):
        mx.mx_gemm_fp8(x.float(), c8, s8, 32, "e8m0")
    with pytest.raises(ValueError):
        mx.mx_gemm_fp8(x, c8[:, :K // 2], s8, 32, "e8m0")
    with pytest.raises(ValueError):
        mx.mx_quantize_fp8(x, 32, "e8m0", codes=torch.zeros((M, K - 1), dtype=u8))
    with pytest.raises(ValueError):
        mx.mx_dequantize_fp8(c8, s8[:-1], 32, "e8m0")
    with pytest.raises(ValueError, match="GPU tensor"):
        mx.mx_gemm_fp8(x, c8, s8, 32, "e8m0")
