"""The hot path captured in a HIP graph: quantize (row-major, tiled and two-level scales),
dequantize, the decode GEMVs (m 1 and 4), the W4A16 and W4A4 products (with a workspace and
with the library's static scratch), the device error split and the tensor statistics, all
recorded once and replayed.  Before every replay the captured input buffers receive new data
(eager work on the same stream) and the device is synchronized; every replay's outputs must
be bit-identical to eager calls on the same inputs.  The library issues no memset or copy of
its own, only kernels, so a captured call is its kernels alone."""
import numpy as np
import pytest
import torch

import microscaling_fp4_weight_amd as mx
import synth
from gpu_util import bf16_dev

pytestmark = pytest.mark.gpu

N, K = 512, 4096
G = 0.0171875  # a per-tensor scale that is not a power of two


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mx.lib()


def _inputs(r):
    w = bf16_dev(synth.normal((N, K), "bf16", f"graph.w.{r}", 0.02, 0.001, 20.0))
    x1 = bf16_dev(synth.normal((1, K), "bf16", f"graph.x1.{r}", 1.0))
    x4 = bf16_dev(synth.normal((4, K), "bf16", f"graph.x4.{r}", 1.0))
    x256 = bf16_dev(synth.normal((256, K), "bf16", f"graph.x256.{r}", 1.0))
    return w, x1, x4, x256


def _run(w, x1, x4, x256, o):
    """The captured sequence: every output goes to a buffer of `o` (nothing is allocated)."""
    mx.mx_quantize(w, 32, "e8m0", codes=o["c"], scales=o["s"])
    mx.mx_quantize(w, 32, "e8m0", layout="tiled", codes=o["ct"], scales=o["st"])
    mx.mx_quantize(w, 32, "ue5m3", G, codes=o["cg"], scales=o["sg"])
    mx.mx_dequantize(o["cg"], o["sg"], K, 32, "ue5m3", G, y=o["deq"])
    mx.mx_gemm(x1, o["c"], o["s"], 32, "e8m0", 1.0, "a16", y=o["y1"])
    mx.mx_gemm(x4, o["c"], o["s"], 32, "e8m0", 1.0, "a16", y=o["y4"])
    mx.mx_gemm(x256, o["cg"], o["sg"], 32, "ue5m3", G, "a16", out_dtype=torch.float32, y=o["y16"])
    mx.mx_gemm(x256, o["ct"], o["st"], 32, "e8m0", 1.0, "a4", layout="tiled", y=o["ya4"], workspace=o["ws"])
    mx.mx_gemm_static(x256, o["c"], o["s"], 32, "e8m0", 1.0, "a4", y=o["ystat"])
    mx.mx_quant_error(w, 32, "e4m3", out=o["err"], workspace=o["wse"])
    mx.mx_tensor_stats(w, out=o["stats"], workspace=o["wss"])


def _buffers(dev):
    u8, bf = torch.uint8, torch.bfloat16
    return {
        "c": torch.empty((N, K // 2), dtype=u8, device=dev),
        "s": torch.empty((N, K // 32), dtype=u8, device=dev),
        "ct": torch.empty((N, K // 2), dtype=u8, device=dev),
        "st": torch.empty(mx.mx_scale_bytes(N, K, 32, "tiled"), dtype=u8, device=dev),
        "cg": torch.empty((N, K // 2), dtype=u8, device=dev),
        "sg": torch.empty((N, K // 32), dtype=u8, device=dev),
        "deq": torch.empty((N, K), dtype=bf, device=dev),
        "y1": torch.empty((1, N), dtype=bf, device=dev),
        "y4": torch.empty((4, N), dtype=bf, device=dev),
        "y16": torch.empty((256, N), dtype=torch.float32, device=dev),
        "ya4": torch.empty((256, N), dtype=bf, device=dev),
        "ystat": torch.empty((256, N), dtype=bf, device=dev),
        "ws": torch.empty(mx.mx_gemm_workspace_size(256, N, K, 32, "a4"), dtype=u8, device=dev),
        "err": torch.zeros(8, dtype=torch.float64, device=dev),
        "wse": torch.empty(max(mx.mx_quant_error_workspace_size(N, K, 32), 16), dtype=u8, device=dev),
        "stats": torch.zeros(4, dtype=torch.float64, device=dev),
        "wss": torch.empty(max(mx.mx_tensor_stats_workspace_size(N, K), 16), dtype=u8, device=dev),
    }


USED = {"err": 7, "stats": 3}  # elements the call writes (the buffers are 16-byte padded)


def _bits(t):
    t = t.detach().cpu()
    return t.view(torch.uint8).numpy().tobytes() if t.dtype != torch.uint8 else t.numpy().tobytes()


def test_hot_path_graph_replays_match_eager():
    dev = torch.device("cuda:0")
    w, x1, x4, x256 = _inputs(0)
    o = _buffers(dev)
    # eager warm-up on a side stream (kernel attributes are set on first use, outside capture)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _run(w, x1, x4, x256, o)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _run(w, x1, x4, x256, o)
    torch.cuda.synchronize()

    prev = None
    for r in range(1, 4):
        nw, nx1, nx4, nx256 = _inputs(r)
        # new data into the captured input buffers, and stale values into every output
        w.copy_(nw)
        x1.copy_(nx1)
        x4.copy_(nx4)
        x256.copy_(nx256)
        for key in ("c", "s", "ct", "st", "cg", "sg"):
            o[key].fill_(0xA5)
        for key in ("deq", "y1", "y4", "y16", "ya4", "ystat", "err", "stats"):
            o[key].fill_(-7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {key: _bits(o[key][:USED.get(key)]) for key in o if not key.startswith("w")}
        # the same calls eagerly on the same inputs, into fresh buffers
        ref = _buffers(dev)
        _run(w, x1, x4, x256, ref)
        torch.cuda.synchronize()
        for key, b in got.items():
            assert b == _bits(ref[key][:USED.get(key)]), f"replay {r}: {key} differs from the eager call"
        # the replay computed on the new inputs: its outputs differ from the previous replay's
        if prev is not None:
            for key in ("c", "y1", "y4", "ya4", "err"):
                assert got[key] != prev[key], f"replay {r}: {key} unchanged by new inputs"
        prev = got
    del graph
