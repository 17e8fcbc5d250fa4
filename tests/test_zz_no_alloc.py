"""mx_gemm_static (the W4A4 workspace in the library's static device buffer) through the C ABI
against mx_gemm with a caller-allocated workspace: the same kernels on the same inputs, so the
outputs must be bit-identical; two calls in a row, the second smaller, so that the second
reads a buffer holding the first call's data.  One case is also checked against the oracle
at the matmul tolerance."""
import ctypes

import numpy as np
import pytest
import torch

import microscaling_fp4_weight_amd as mx
import oracle
import synth
from gpu_util import DEV, assert_gemm_close, bf16_dev, to_host_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mx.lib()


def _case(m, n, k, tag):
    x = synth.normal((m, k), "bf16", f"na.x.{tag}", 1.0)
    w = synth.normal((n, k), "bf16", f"na.w.{tag}", 0.015, 0.001, 20.0)
    return x, w


def _static(L, xd, c, s, m, n, k, layout, mode, y):
    sp = torch.cuda.current_stream().cuda_stream
    return L.mx_gemm_static(xd.data_ptr(), m, n, k, k, c.data_ptr(), s.data_ptr(), 32, mx.FMT["e8m0"], 1.0,
                            mx.LAYOUT[layout], mx.MODE[mode], y.data_ptr(), 1 if y.dtype == torch.bfloat16 else 0,
                            n, sp)


@pytest.mark.parametrize("layout", ["rowmajor", "tiled"])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_static_matches_workspace_entry_point(layout, out):
    L = mx.lib()
    for (m, n, k), tag in (((512, 1024, 2048), "big"), ((100, 320, 512), "small")):
        print(f"no-alloc gemm {layout} {out} m={m} n={n} k={k}", flush=True)
        x, w = _case(m, n, k, tag)
        xd, wd = bf16_dev(x), bf16_dev(w)
        c, s = mx.mx_quantize(wd, 32, "e8m0", layout=layout)
        y_ref = mx.mx_gemm(xd, c, s, 32, "e8m0", 1.0, "a4", out_dtype=out, layout=layout)
        y = torch.full((m, n), float("nan"), dtype=out, device=DEV)
        st = _static(L, xd, c, s, m, n, k, layout, "a4", y)
        assert st == 0, mx.mx_status_string(st)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_host_bits(y), to_host_bits(y_ref))
        if tag == "small" and out == torch.float32:
            rc, rs = oracle.quantize(w, 32, "e8m0")
            yref, aref = oracle.gemm(x, rc, rs, 32, "e8m0", 1.0, "a4")
            assert_gemm_close(to_host_bits(y), yref, aref, False, f"static a4 {layout}")


def test_static_w4a16_and_python_wrapper():
    m, n, k = 4, 256, 1024
    x, w = _case(m, n, k, "a16")
    xd, wd = bf16_dev(x), bf16_dev(w)
    c, s = mx.mx_quantize(wd, 32, "e8m0")
    y_ref = mx.mx_gemm(xd, c, s, 32, "e8m0", 1.0, "a16", out_dtype=torch.float32)
    y = torch.empty((m, n), dtype=torch.float32, device=DEV)
    mx.mx_gemm_static(xd, c, s, 32, "e8m0", 1.0, "a16", y=y)
    y4 = torch.empty((m, n), dtype=torch.float32, device=DEV)
    mx.mx_gemm_static(xd, c, s, 32, "e8m0", 1.0, "a4", y=y4)
    y4_ref = mx.mx_gemm(xd, c, s, 32, "e8m0", 1.0, "a4", out_dtype=torch.float32)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host_bits(y), to_host_bits(y_ref))
    np.testing.assert_array_equal(to_host_bits(y4), to_host_bits(y4_ref))


def test_static_rejects_oversized_call_on_host():
    L = mx.lib()
    m, n, k = 8192, 256, 16384  # activations alone need 64 MiB
    assert mx.mx_gemm_workspace_size(m, n, k, 32, "a4") > mx.GEMM_STATIC_SCRATCH_BYTES
    fake = 1 << 20  # never dereferenced: the size check comes first
    st = L.mx_gemm_static(fake, m, n, k, k, fake, fake, 32, mx.FMT["e8m0"], 1.0, 0, mx.MODE["a4"], fake, 0, n,
                          ctypes.c_void_p(None))
    assert st == -5 and "static scratch" in mx.mx_status_string(st)
