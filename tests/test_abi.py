"""C-ABI checks that need no GPU: libmx.so loads, exports exactly what include/mx.h declares,
and rejects invalid arguments on the host with the documented status (nothing is launched
on these paths)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mx.h")

OK, INVALID, UNSUPPORTED, ALIGN = 0, -1, -2, -3
E4M3, UE5M3, E8M0 = 0, 1, 2
F32, BF16 = 0, 1
A16, A4 = 0, 1


@pytest.fixture(scope="module")
def L():
    import microscaling_fp4_weight_amd as mx
    return mx.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(mx_\w+)\s*\(", text, re.M)))


def test_exports_match_header(L):
    names = declared_functions()
    assert names == ["mx_adaptive_block_size", "mx_dequantize", "mx_dequantize_fp8", "mx_gemm",
                     "mx_gemm_fp8", "mx_gemm_static", "mx_gemm_workspace_size", "mx_layer_block_size", "mx_quant_error",
                     "mx_quant_error_workspace_size", "mx_quantize", "mx_quantize_fp8", "mx_scale_bytes",
                     "mx_status_string", "mx_tensor_stats", "mx_tensor_stats_workspace_size",
                     "mx_use_fp8"]
    for n in names:
        assert hasattr(L, n)
    so = os.path.join(ROOT, "microscaling_fp4_weight_amd", "libmx.so")
    out = subprocess.run(["nm", "-D", "--defined-only", so], capture_output=True, text=True).stdout
    exported = sorted(set(re.findall(r" T (mx_\w+)$", out, re.M)))
    assert exported == names


def test_status_strings(L):
    for s in (OK, INVALID, UNSUPPORTED, ALIGN, -4, -5):
        assert L.mx_status_string(s)
    assert L.mx_status_string(OK) == b"success"


FAKE = 1 << 20  # a 16-byte aligned non-null address; never dereferenced on these paths


@pytest.mark.parametrize("args,status", [
    # (x, x_type, rows, k, ld_x, block, fmt, g, layout, codes, scales) -> status
    ((FAKE, BF16, 4, 33, 33, 32, E8M0, 1.0, 0, FAKE, FAKE), INVALID),     # k odd / k % block
    ((FAKE, BF16, 4, 48, 48, 32, E8M0, 1.0, 0, FAKE, FAKE), INVALID),     # k % block
    ((FAKE, BF16, 4, 64, 64, 12, E8M0, 1.0, 0, FAKE, FAKE), INVALID),     # block not listed
    ((FAKE, BF16, 4, 64, 64, 512, E8M0, 1.0, 0, FAKE, FAKE), INVALID),
    ((FAKE, BF16, -1, 64, 64, 32, E8M0, 1.0, 0, FAKE, FAKE), INVALID),    # negative rows
    ((FAKE, BF16, 4, 64, 32, 32, E8M0, 1.0, 0, FAKE, FAKE), INVALID),     # ld < k
    ((FAKE, 7, 4, 64, 64, 32, E8M0, 1.0, 0, FAKE, FAKE), INVALID),        # dtype
    ((FAKE, BF16, 4, 64, 64, 32, 3, 1.0, 0, FAKE, FAKE), INVALID),        # fmt
    ((FAKE, BF16, 4, 64, 64, 32, E8M0, 1.0, 3, FAKE, FAKE), INVALID),     # layout
    ((FAKE, BF16, 4, 64, 64, 16, E8M0, 1.0, 2, FAKE, FAKE), UNSUPPORTED), # preshuffled needs block 32
    ((FAKE, BF16, 4, 64, 64, 16, E8M0, 1.0, 1, FAKE, FAKE), UNSUPPORTED), # tiled needs block 32
    ((FAKE, BF16, 4, 1 << 23, 1 << 23, 32, E8M0, 1.0, 1, FAKE, FAKE), UNSUPPORTED),  # tiled k bound
    ((FAKE, BF16, 4, 64, 64, 32, E8M0, 0.0, 0, FAKE, FAKE), INVALID),     # g = 0
    ((FAKE, BF16, 4, 64, 64, 32, E8M0, -1.0, 0, FAKE, FAKE), INVALID),    # g < 0
    ((FAKE, BF16, 4, 64, 64, 32, E8M0, float("inf"), 0, FAKE, FAKE), INVALID),
    ((FAKE, BF16, 4, 64, 64, 32, E8M0, float("nan"), 0, FAKE, FAKE), INVALID),
    ((FAKE, BF16, 4, 64, 64, 32, E8M0, 1e-40, 0, FAKE, FAKE), INVALID),   # subnormal g
    ((None, BF16, 4, 64, 64, 32, E8M0, 1.0, 0, FAKE, FAKE), INVALID),     # null x
    ((FAKE, BF16, 4, 64, 64, 32, E8M0, 1.0, 0, None, FAKE), INVALID),
    ((FAKE, BF16, 4, 64, 64, 32, E8M0, 1.0, 0, FAKE, None), INVALID),
    ((FAKE + 8, BF16, 4, 64, 64, 32, E8M0, 1.0, 0, FAKE, FAKE), ALIGN),   # misaligned
    ((FAKE, BF16, 4, 64, 64, 32, E8M0, 1.0, 0, FAKE + 1, FAKE), ALIGN),
    ((None, BF16, 0, 64, 64, 32, E8M0, 1.0, 0, None, None), OK),          # empty: no launch
    ((None, BF16, 5, 0, 0, 32, E8M0, 1.0, 0, None, None), OK),
])
def test_quantize_validation(L, args, status):
    assert L.mx_quantize(*args, None) == status


def test_dequantize_validation(L):
    # (codes, scales, rows, k, block, fmt, g, layout, y, y_type, ld_y)
    assert L.mx_dequantize(FAKE, FAKE, 4, 64, 32, E8M0, 1.0, 0, FAKE, 9, 64, None) == INVALID
    assert L.mx_dequantize(FAKE, FAKE, 4, 64, 32, E8M0, 1.0, 0, FAKE, F32, 63, None) == INVALID
    assert L.mx_dequantize(FAKE, FAKE, 4, 60, 8, E8M0, 1.0, 0, FAKE, F32, 64, None) == INVALID
    assert L.mx_dequantize(FAKE, None, 4, 64, 32, E8M0, 1.0, 0, FAKE, F32, 64, None) == INVALID
    assert L.mx_dequantize(FAKE, FAKE, 4, 64, 32, E8M0, 1.0, 0, FAKE + 4, F32, 64, None) == ALIGN
    assert L.mx_dequantize(None, None, 0, 64, 32, E8M0, 1.0, 0, None, F32, 64, None) == OK


def test_scale_bytes(L):
    sb = L.mx_scale_bytes
    assert sb(4, 64, 32, 0) == 8
    assert sb(5, 96, 4, 0) == 5 * 24
    # tiled: ceil(rows / 256) * ceil(k / 256) * 2048
    assert sb(4, 64, 32, 1) == 2048
    assert sb(300, 8192, 32, 1) == 2 * 32 * 2048
    assert sb(256, 4224, 32, 1) == 1 * 17 * 2048
    assert sb(0, 64, 32, 1) == 0
    assert sb(4, 64, 16, 1) == 0          # tiled is defined for block 32 only
    assert sb(4, 48, 32, 0) == 0          # k % block
    # preshuffled: ceil(rows / 8) * ceil(k / 2048) * 512
    assert sb(4, 64, 32, 2) == 512
    assert sb(9, 4224, 32, 2) == 2 * 3 * 512
    assert sb(8, 2048, 32, 2) == 512
    assert sb(4, 64, 16, 2) == 0          # preshuffled is defined for block 32 only
    assert sb(4, 64, 32, 3) == 0          # unknown layout


def test_gemm_validation_and_workspace(L):
    ws = L.mx_gemm_workspace_size
    assert ws(2048, 28672, 8192, 32, A16) == 0
    assert ws(2048, 28672, 8192, 32, A4) == 2048 * 4096 + 2048 * 256
    assert ws(3, 5, 64, 32, A4) == 256 + 2048  # codes rounded to 256 bytes; one tiled scale block
    assert ws(300, 5, 4224, 32, A4) == 300 * 2112 + 2 * 17 * 2048
    assert ws(3, 5, 64, 16, A4) == 0          # W4A4 needs block 32
    assert ws(3, 5, 63, 32, A4) == 0

    def gemm(m=4, n=8, k=64, ldx=64, block=32, fmt=E8M0, g=1.0, mode=A16, yt=F32, ldy=8,
             work=None, wbytes=0, x=FAKE, wc=FAKE, wsc=FAKE, y=FAKE, layout=0):
        return L.mx_gemm(x, m, n, k, ldx, wc, wsc, block, fmt, g, layout, mode, y, yt, ldy, work,
                         wbytes, None)

    # tiled weight scales: W4A4 matrix-core path only (k % 128 == 0)
    assert gemm(layout=1) == UNSUPPORTED                                    # W4A16
    assert gemm(layout=1, mode=A4, work=FAKE, wbytes=1 << 20) == UNSUPPORTED  # k = 64
    assert gemm(layout=1, mode=A4, block=16, k=128, ldx=128) == UNSUPPORTED
    assert gemm(layout=3) == INVALID
    # preshuffled weight scales: the m = 1 W4A16 GEMV only
    assert gemm(layout=2) == UNSUPPORTED                                    # m = 4
    assert gemm(layout=2, m=1, mode=A4, work=FAKE, wbytes=1 << 20) == UNSUPPORTED
    assert gemm(layout=2, m=1, ldx=68) == UNSUPPORTED                       # ld_x not a multiple of 8
    assert gemm(layout=2, m=1, block=16) == UNSUPPORTED

    assert gemm(mode=A4, fmt=E4M3) == UNSUPPORTED      # W4A4 is E8M0-only
    assert gemm(mode=A4, block=64) == UNSUPPORTED      # and block 32 only
    assert gemm(mode=A4, work=FAKE, wbytes=100) == INVALID   # workspace too small
    assert gemm(mode=A4, work=None, wbytes=0) == INVALID
    assert gemm(ldy=7) == INVALID
    assert gemm(ldx=63) == INVALID
    assert gemm(k=48) == INVALID                       # k % block
    assert gemm(mode=2) == INVALID
    assert gemm(yt=5) == INVALID
    assert gemm(g=0.0) == INVALID
    assert gemm(y=None) == INVALID
    assert gemm(y=FAKE + 2) == ALIGN
    assert gemm(wsc=FAKE + 8) == ALIGN
    assert gemm(m=0, x=None, y=None) == OK
    assert gemm(n=0, wc=None, wsc=None, y=None) == OK
    assert gemm(k=0, y=FAKE + 2) == ALIGN


def test_quant_error_validation(L):
    ws = L.mx_quant_error_workspace_size
    assert ws(4, 64, 32) == 256            # one workgroup: 6 doubles, rounded to 256 bytes
    assert ws(4096, 11008, 4) == 1024 * 6 * 8  # the grid is capped at 1024 workgroups
    assert ws(0, 64, 32) == 0
    assert ws(4, 48, 32) == 0              # k % block

    def qe(x=FAKE, xt=BF16, rows=4, k=64, ldx=64, block=32, fmt=E8M0, g=1.0, xh=None, ldh=0,
           out=FAKE, work=FAKE, wbytes=256):
        return L.mx_quant_error(x, xt, rows, k, ldx, block, fmt, g, xh, ldh, out, work, wbytes,
                                None)

    assert qe(out=None) == INVALID
    assert qe(work=None) == INVALID
    assert qe(wbytes=255) == INVALID
    assert qe(block=12) == INVALID
    assert qe(fmt=3) == INVALID
    assert qe(xt=7) == INVALID
    assert qe(ldx=63) == INVALID
    assert qe(g=0.0) == INVALID
    assert qe(xh=FAKE, ldh=63) == INVALID    # x_hat row stride below k
    assert qe(xh=FAKE + 4, ldh=64) == ALIGN
    assert qe(out=FAKE + 8) == ALIGN
    assert qe(x=FAKE + 2) == ALIGN
    assert qe(rows=0, x=None, out=None, work=None, wbytes=0) == OK  # empty: nothing launched


def test_block_size_policy_matches_oracle(L):
    import oracle
    for sigma in (0.0, 0.005, 0.00999999, 0.01, 0.02, 0.0999999, 0.1, 0.118, 2.0, float("nan"),
                  float("inf")):
        assert L.mx_adaptive_block_size(sigma) == oracle.adaptive_block_size(sigma), sigma
    for i, kind in enumerate(("qkv", "ffn_gate_up", "output")):
        assert L.mx_layer_block_size(i) == oracle.layer_block_size(kind)
    assert L.mx_layer_block_size(3) == 0 and L.mx_layer_block_size(-1) == 0


def test_tensor_stats_validation(L):
    ws = L.mx_tensor_stats_workspace_size
    assert ws(4, 64) == 256                   # one workgroup: 2 doubles, rounded up
    assert ws(4096, 11008) == 1024 * 2 * 8    # capped grid
    assert ws(0, 64) == 0

    def ts(x=FAKE, xt=BF16, rows=4, k=64, ldx=64, out=FAKE, work=FAKE, wbytes=256):
        return L.mx_tensor_stats(x, xt, rows, k, ldx, out, work, wbytes, None)

    assert ts(ldx=63) == INVALID
    assert ts(rows=-1) == INVALID
    assert ts(xt=5) == INVALID
    assert ts(out=None) == INVALID
    assert ts(work=None) == INVALID
    assert ts(wbytes=255) == INVALID
    assert ts(x=FAKE + 4) == ALIGN
    assert ts(out=FAKE + 8) == ALIGN
    assert ts(rows=0, x=None, out=None, work=None, wbytes=0) == OK
    assert ts(rows=1 << 20, k=1 << 15, ldx=1 << 15, wbytes=1 << 20) == UNSUPPORTED


def test_fp8_validation(L):
    import oracle
    for sigma in (0.0, 5e-5, 9.99e-5, 1e-4, 0.02, float("nan")):
        assert L.mx_use_fp8(sigma) == int(oracle.use_fp8(sigma))
    q = L.mx_quantize_fp8
    assert q(FAKE, BF16, 4, 48, 48, 32, E8M0, 1.0, FAKE, FAKE, None) == INVALID   # k % block
    assert q(FAKE, BF16, 4, 64, 63, 32, E8M0, 1.0, FAKE, FAKE, None) == INVALID   # ld < k
    assert q(FAKE, 7, 4, 64, 64, 32, E8M0, 1.0, FAKE, FAKE, None) == INVALID
    assert q(FAKE, BF16, 4, 64, 64, 32, 3, 1.0, FAKE, FAKE, None) == INVALID
    assert q(FAKE, BF16, 4, 64, 64, 32, E8M0, 0.0, FAKE, FAKE, None) == INVALID
    assert q(None, BF16, 4, 64, 64, 32, E8M0, 1.0, FAKE, FAKE, None) == INVALID
    assert q(FAKE + 2, BF16, 4, 64, 64, 32, E8M0, 1.0, FAKE, FAKE, None) == ALIGN
    assert q(None, BF16, 0, 64, 64, 32, E8M0, 1.0, None, None, None) == OK
    d = L.mx_dequantize_fp8
    assert d(FAKE, FAKE, 4, 64, 32, E8M0, 1.0, FAKE, 9, 64, None) == INVALID
    assert d(FAKE, FAKE, 4, 64, 32, E8M0, 1.0, FAKE, F32, 63, None) == INVALID
    assert d(FAKE, FAKE, 4, 64, 32, E8M0, 1.0, FAKE + 4, F32, 64, None) == ALIGN
    assert d(None, None, 0, 64, 32, E8M0, 1.0, None, F32, 64, None) == OK
    gm = L.mx_gemm_fp8
    assert gm(FAKE, 4, 8, 48, 48, FAKE, FAKE, 32, E8M0, 1.0, FAKE, F32, 8, None) == INVALID  # k % block
    assert gm(FAKE, 4, 8, 64, 63, FAKE, FAKE, 32, E8M0, 1.0, FAKE, F32, 8, None) == INVALID
    assert gm(FAKE, 4, 8, 64, 64, FAKE, FAKE, 32, E8M0, 1.0, FAKE, F32, 7, None) == INVALID
    assert gm(FAKE, 4, 8, 64, 64, FAKE, FAKE, 32, E8M0, 1.0, None, F32, 8, None) == INVALID
    assert gm(FAKE, 4, 8, 64, 64, FAKE, FAKE + 8, 32, E8M0, 1.0, FAKE, F32, 8, None) == ALIGN
    assert gm(FAKE, -1, 8, 64, 64, FAKE, FAKE, 32, E8M0, 1.0, FAKE, F32, 8, None) == INVALID
    assert gm(None, 0, 8, 64, 64, None, None, 32, E8M0, 1.0, None, F32, 8, None) == OK
