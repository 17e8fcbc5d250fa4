#!/usr/bin/env python3
"""Benchmark of the MX FP4 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-rows] [--no-cpu]
    python bench.py --pmc-run      # launches for rocprofv3 --pmc traffic counters (see below)
    python bench.py --pmc-run rows # launches of the GEMV / GEMM rows for rocprofv3 --pmc
    python bench.py --pmc-run c5   # launches of the 405B-FFN W4A16 products for rocprofv3 --pmc

One step = the whole block-size/scale sweep on the Llama-7B FFN-shaped weight
(4096 x 11008 bf16 ~ N(0, sigma^2), 0.1% entries x20): for every sigma in {0.005, 0.02, 0.1},
block in {4, 8, 16, 32, 64, 128, 256} and scale format in {E4M3, UE5M3, E8M0}, one MX quantize
(bf16 -> codes + scales) and one dequantize (codes + scales -> bf16): 126 launches.  Inputs
and outputs rotate over > 512 MB of distinct buffers so every launch reads HBM, not the
256 MB Infinity Cache.  `value` is the algorithmic bytes of a step divided by its time.

The remaining rows of the hot path are measured in the same run (`rows`): decode GEMV
(M in {1,4,16}, K 4096, N in {4096, 14336}, block 32 E8M0, bf16 out, back-to-back over
distinct weight copies), 70B-FFN prefill GEMM (2048 x 8192 x 28672) in W4A16 and W4A4, and
the 405B-FFN shapes with two-level UE5M3 scaling (offline weight quantize; GEMV M=1; GEMM
M=256, 4096).  `roofline` is for the dominant kernel, the B=32 E8M0 quantize; `cpu_baseline`
times the single-threaded CPU oracle, pinned to one core, on a bounded sample of the same
sweep and on samples of the GEMV / GEMM rows.

Prints ONE short JSON line on stdout (the summary: value, roofline, cpu_baseline and the rows
as time and fraction of roofline); progress and the full per-configuration record
(`[bench] detail {...}`: per-config times, the device error split, the block-size policy, the
FP8 fallback rows) go to stderr, and with `--detail PATH` also to a JSON file.

`--pmc-run` only launches the dominant kernel (five times) and a plain device copy of known
size (five times, the calibration for the HBM byte counters), for
`rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE`; the resulting per-launch bytes are kept in
profiles/traffic.json and reported as `roofline.traffic` while the kernel source is unchanged.
`--pmc-run rows` launches the decode GEMV (m 1, 4, 16; n 14336), the 405B-FFN GEMV (m 1), the 70B-FFN
prefill GEMM in W4A16 and W4A4 (tiled weight scales) three times each, and the same copy, for
the HBM byte and matrix-core counters of those kernels; `--pmc-run c5` launches the 405B-FFN
W4A16 products (m 256 and 4096) three times each.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MX quantize GB/s; MXFP4 GEMV/GEMM TFLOP/s (% of HBM / MFMA roofline)"
PEAK_HBM = 8.0e12          # B/s, MI355X HBM3E
PEAK_BF16 = 2.5e15         # dense bf16 MFMA FLOP/s
PEAK_FP4 = 10.1e15         # dense fp4 MFMA FLOP/s
FMTS = ("e4m3", "ue5m3", "e8m0")
BLOCKS = (4, 8, 16, 32, 64, 128, 256)
SIGMAS = (0.005, 0.02, 0.1)
C2_ROWS, C2_K = 4096, 11008


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def quant_bytes(n: int, block: int, in_bytes: int = 2) -> int:
    """Algorithmic HBM bytes of one quantize (or dequantize to the same dtype) of n elements:
    read the dense tensor, write n/2 code bytes and n/block scale bytes."""
    return n * in_bytes + n // 2 + n // block


def gemv_bytes(m: int, n: int, k: int, block: int) -> int:
    return n * k // 2 + n * k // block + 2 * m * k + 2 * m * n


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 2000 steps of 2.65 ms: about 5 s of timed GPU work, long enough for an outside
    # utilisation sampler to see it
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-rows", action="store_true", help="skip the GEMV/GEMM rows")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--detail", default=None,
                    help="also write the full per-configuration record to this JSON file")
    ap.add_argument("--library-ref", action="store_true",
                    help="only time the vendor library's bf16 and MXFP4 GEMMs at the 70B-FFN "
                         "shape beside this library's W4A16 and W4A4 modes (one JSON line)")
    ap.add_argument("--pmc-run", nargs="?", const="quantize", choices=("quantize", "rows", "c5"),
                    help="only the launches that the counters are read on: the dominant kernel "
                         "(default), the GEMV / GEMM rows, or the 405B-FFN W4A16 products")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the hot path runs on a single MI355X and this "
              "library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import microscaling_fp4_weight_amd as mx
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = mx.lib()
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    if args.pmc_run == "quantize":
        pmc_run(mx, torch, np, synth, dev)
        return
    if args.pmc_run == "rows":
        pmc_rows(mx, torch, np, synth, dev)
        return
    if args.pmc_run == "c5":
        pmc_c5(mx, torch, np, synth, dev)
        return
    if args.library_ref:
        library_ref(mx, torch, np, synth, dev, stream)
        return

    # ---------------------------------------------------------------- C2 sweep setup
    t0 = time.time()
    inputs = []
    for sigma in SIGMAS:
        w = synth.c2_weight(sigma)
        wd = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to(dev)
        inputs.append(wd)
        inputs.append(wd.clone())  # two copies per sigma: six 90 MB inputs in rotation
    n = C2_ROWS * C2_K
    sweep_cfgs = [(si, b, f) for b in BLOCKS for f in FMTS for si in range(len(SIGMAS))]
    codes = [torch.empty((C2_ROWS, C2_K // 2), dtype=torch.uint8, device=dev) for _ in sweep_cfgs]
    scales = [torch.empty((C2_ROWS, C2_K // b), dtype=torch.uint8, device=dev) for (_, b, _) in sweep_cfgs]
    deq_out = [torch.empty((C2_ROWS, C2_K), dtype=torch.bfloat16, device=dev) for _ in range(6)]
    log(f"C2 setup {time.time() - t0:.1f}s: {len(sweep_cfgs)} configurations")

    qcalls, dcalls = [], []
    step_bytes = 0
    for i, (si, b, f) in enumerate(sweep_cfgs):
        x = inputs[2 * si + (i // len(SIGMAS)) % 2]
        qcalls.append((x.data_ptr(), 1, C2_ROWS, C2_K, C2_K, b, mx.FMT[f], 1.0, 0,
                       codes[i].data_ptr(), scales[i].data_ptr(), sp))
        dcalls.append((codes[i].data_ptr(), scales[i].data_ptr(), C2_ROWS, C2_K, b, mx.FMT[f], 1.0,
                       0, deq_out[i % 6].data_ptr(), 1, C2_K, sp))
        step_bytes += 2 * quant_bytes(n, b)
    # the dominant kernel's three launches (one per sigma) are consecutive in the step; one
    # event pair around them gives its average launch duration inside the timed region
    dom = [i for i, c in enumerate(sweep_cfgs) if c[1] == 32 and c[2] == "e8m0"]
    assert dom == list(range(dom[0], dom[0] + len(SIGMAS)))
    q, dq = L.mx_quantize, L.mx_dequantize

    def step(ev=None):
        for i, c in enumerate(qcalls):
            if ev is not None and i == dom[0]:
                ev[0].record(stream)
            st = q(*c)
            if ev is not None and i == dom[-1]:
                ev[1].record(stream)
            if st:
                raise mx.MXError(st, "mx_quantize")
        for c in dcalls:
            st = dq(*c)
            if st:
                raise mx.MXError(st, "mx_dequantize")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    dom_events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    start.record(stream)
    for s in range(args.steps):
        step(dom_events[s])
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    gpu_ms = start.elapsed_time(end)
    ms_per_step = max(gpu_ms, wall * 1e3) / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    dom_ms = sorted(a.elapsed_time(b) / len(dom) for a, b in dom_events)
    dom_avg_ms = sum(dom_ms) / len(dom_ms)
    dom_bytes = quant_bytes(n, 32)
    log(f"C2 sweep: {ms_per_step:.3f} ms/step, {value:.0f} GB/s; dominant kernel avg {dom_avg_ms * 1e3:.2f} us")

    # per-config kernel times (one event pair per launch, outside the timed steps)
    per_cfg = {}
    for kind, calls, fn in (("quantize", qcalls, q), ("dequantize", dcalls, dq)):
        evs = []
        for rep in range(3):
            for i, c in enumerate(calls):
                a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                fn(*c)
                b_.record(stream)
                evs.append((i, a, b_))
        torch.cuda.synchronize()
        acc = {}
        for i, a, b_ in evs:
            acc.setdefault(i, []).append(a.elapsed_time(b_))
        for i, ts in acc.items():
            si, b, f = sweep_cfgs[i]
            key = f"{kind}.B{b}.{f}"
            per_cfg.setdefault(key, []).append(min(ts))
    per_config = {}
    for key, ts in per_cfg.items():
        b = int(key.split(".")[1][1:])
        t = sorted(ts)[len(ts) // 2]
        gbs = quant_bytes(n, b) / (t * 1e-3) / 1e9
        per_config[key] = {"us": round(t * 1e3, 2), "GB/s": round(gbs, 1),
                           "frac_hbm": round(gbs * 1e9 / PEAK_HBM, 3)}

    # traffic counters (rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE), taken from the committed
    # profile when the quantize kernel's source has not changed since it was measured
    traffic = load_traffic("quantize")

    roofline = {"bound": "hbm", "kernel": "quantize_fast_kernel<32, E8M0, bf16, g=1>",
                "achieved": round(dom_bytes / (dom_avg_ms * 1e-3) / 1e9, 1),
                "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                "frac": round(dom_bytes / (dom_avg_ms * 1e-3) / PEAK_HBM, 4),
                "traffic": traffic, "bytes_per_launch": dom_bytes,
                "avg_launch_us": round(dom_avg_ms * 1e3, 3)}

    error_split = measure_error_split(mx, L, torch, inputs, sweep_cfgs, dev, stream)
    block_policy = measure_block_policy(mx, torch, inputs, error_split, dev, stream)

    # free the sweep buffers before the GEMM rows
    del inputs, codes, scales, deq_out, qcalls, dcalls
    torch.cuda.empty_cache()

    rows = None if args.no_rows else measure_rows(mx, L, torch, np, synth, dev, stream)
    fp8 = None if args.no_rows else measure_fp8(mx, L, torch, np, synth, dev, stream)

    detail = {"per_config": per_config, "error_split": error_split, "block_policy": block_policy,
              "rows": rows, "fp8_fallback": fp8}
    cpu = None if args.no_cpu else cpu_baseline(np, synth, value, rows)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama7b-ffn 4096x11008 bf16 block/scale sweep: 3 sigma x 7 blocks "
                               "x 3 scale formats, quantize + dequantize (126 launches/step)",
                   "bytes_per_step": step_bytes},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "rows": compact_rows(rows, fp8, error_split),
    }
    line = json.dumps(out, separators=(",", ":"))
    # the full per-configuration record goes to stderr (and to --detail if given); stdout
    # carries one short line
    dline = json.dumps(detail, separators=(",", ":"))
    log("detail " + dline)
    if args.detail:
        os.makedirs(os.path.dirname(os.path.abspath(args.detail)), exist_ok=True)
        with open(args.detail, "w") as fh:
            fh.write(json.dumps({"summary": out, **detail}, indent=1))
    if len(line) > 4096:
        log(f"warning: summary line is {len(line)} bytes")
    print(line, flush=True)


def compact_rows(rows, fp8, error_split):
    """The GEMV / GEMM / 405B rows in short form: time per launch (us for the GEMVs, ms
    otherwise) and the fraction of the roofline that bounds the row ("of": HBM for quantize and
    the GEMVs, the bf16 or FP4 matrix-core peak for the GEMMs)."""
    if rows is None:
        return None
    out = {}

    def put(name, r, fkey, of):
        if r is None:
            return
        if "us_per_launch" in r:
            out[name] = {"us": r["us_per_launch"], "frac": r[fkey], "of": of}
        elif "us" in r:
            out[name] = {"us": r["us"], "frac": r[fkey], "of": of}
        else:
            out[name] = {"ms": r["ms"], "frac": r[fkey], "of": of}

    for nn in (4096, 14336):
        for m in (1, 4, 16):
            key = f"gemv_a16.m{m}.n{nn}.k4096"
            put(key, rows.get(key), "frac_hbm", "hbm")
    for key, of in (("gemm_a16.m2048.n28672.k8192", "bf16"), ("gemm_a4.m2048.n28672.k8192", "fp4"),
                    ("gemm_a4.m2048.n28672.k8192.tiled_scales", "fp4")):
        put(key, rows.get(key), "frac_peak", of)
    put("quantize.ue5m3.g.n53248.k16384", rows.get("quantize.ue5m3.g.n53248.k16384"), "frac_hbm", "hbm")
    for key in ("gemm_a16.ue5m3.g.m1.n53248.k16384", "gemm_a16.ue5m3.g.m1.n53248.k16384.preshuffled_scales"):
        put(key.replace("gemm_a16", "gemv_a16"), rows.get(key), "frac_hbm", "hbm")
    for m in (256, 4096):
        key = f"gemm_a16.ue5m3.g.m{m}.n53248.k16384"
        put(key, rows.get(key), "frac_peak_bf16", "bf16")
    if error_split is not None:
        out["error_split.63cfg"] = {"ms": error_split["sweep_ms"],
                                    "frac": round(error_split["sweep_GB/s"] * 1e9 / PEAK_HBM, 3), "of": "hbm"}
    for key, r in (fp8 or {}).items():
        put(key, r, "frac_peak_bf16" if key.startswith("gemm_w8") else "frac_hbm",
            "bf16" if key.startswith("gemm_w8") else "hbm")
    return out


def measure_error_split(mx, L, torch, inputs, sweep_cfgs, dev, stream):
    """The sweep's error split computed on the device (mx_quant_error: quantize, dequantize and
    the fp64 MSE_elem / MSE_max / MSE_zero sums in one pass over the weight): per-config
    kernel time (median of 3, one event pair per launch), the whole 63-config sweep, and the
    device MSE terms; plus the fake-quant variant that also writes x^ (block 32, E4M3)."""
    n = C2_ROWS * C2_K
    sp = stream.cuda_stream
    need = max(mx.mx_quant_error_workspace_size(C2_ROWS, C2_K, b) for b in BLOCKS)
    work = torch.empty(need, dtype=torch.uint8, device=dev)
    outs = torch.zeros((len(sweep_cfgs), 8), dtype=torch.float64, device=dev)
    calls = []
    for i, (si, b, f) in enumerate(sweep_cfgs):
        x = inputs[2 * si + (i // len(SIGMAS)) % 2]
        calls.append((x.data_ptr(), 1, C2_ROWS, C2_K, C2_K, b, mx.FMT[f], 1.0, None, 0,
                       outs[i].data_ptr(), work.data_ptr(), need, sp))
    qe = L.mx_quant_error

    def run(c):
        st = qe(*c)
        if st:
            raise mx.MXError(st, "mx_quant_error")

    for c in calls:  # warm-up
        run(c)
    a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for c in calls:
        run(c)
    b_.record(stream)
    evs = []
    for rep in range(3):
        for i, c in enumerate(calls):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run(c)
            e1.record(stream)
            evs.append((i, e0, e1))
    # fake quantization: the error split plus x^ written (sigma 0.02, block 32, E4M3)
    fi = sweep_cfgs.index((1, 32, "e4m3"))
    xh = torch.empty((C2_ROWS, C2_K), dtype=torch.bfloat16, device=dev)
    fq = list(calls[fi])
    fq[8], fq[9] = xh.data_ptr(), C2_K
    run(fq)
    fevs = []
    for rep in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run(fq)
        e1.record(stream)
        fevs.append((e0, e1))
    torch.cuda.synchronize()
    sweep_ms = a.elapsed_time(b_)
    acc = {}
    for i, e0, e1 in evs:
        acc.setdefault(i, []).append(e0.elapsed_time(e1))
    vals = outs.cpu().numpy()
    per = {}
    for i, ts in acc.items():
        si, b, f = sweep_cfgs[i]
        t = sorted(ts)[1]
        gbs = 2 * n / (t * 1e-3) / 1e9
        per[f"s{SIGMAS[si]}.B{b}.{f}"] = {
            "us": round(t * 1e3, 2), "GB/s": round(gbs, 1), "frac_hbm": round(gbs * 1e9 / PEAK_HBM, 3),
            "mse_elem": float(vals[i, 0]), "mse_max": float(vals[i, 1]), "mse_zero": float(vals[i, 2]),
            "mse_total": float(vals[i, 3]),
            "flushed_blocks": int(vals[i, 5])}
    ft = sorted(e0.elapsed_time(e1) for e0, e1 in fevs)[2]
    fgbs = 4 * n / (ft * 1e-3) / 1e9
    log(f"error split: 63-config sweep {sweep_ms:.3f} ms; B32 E4M3 {per['s0.02.B32.e4m3']['us']} us; "
        f"fake quant {ft * 1e3:.1f} us")
    return {"kernel": "quant_error_fast_kernel", "bytes_per_launch": 2 * n,
            "sweep_ms": round(sweep_ms, 3),
            "sweep_GB/s": round(2 * n * len(calls) / (sweep_ms * 1e-3) / 1e9, 1),
            "fake_quant.s0.02.B32.e4m3": {"us": round(ft * 1e3, 2), "bytes": 4 * n, "GB/s": round(fgbs, 1),
                                          "frac_hbm": round(fgbs * 1e9 / PEAK_HBM, 3)},
            "per_config": per}


def measure_fp8(mx, L, torch, np, synth, dev, stream):
    """The FP8 weight fallback: E4M3-element quantize / dequantize of the Llama-7B FFN weight
    (block 32, E8M0), the W8A16 decode GEMV (distinct weights back to back, graph replay, as
    the W4A16 rows) and the 70B-FFN prefill GEMM."""
    res = {}
    bf = torch.bfloat16

    def dev_bf16(a):
        return torch.from_numpy(a.view(np.int16)).view(bf).to(dev)

    n = C2_ROWS * C2_K
    ws = [dev_bf16(synth.c2_weight(0.02))]
    ws.append(ws[0].clone())
    ws.append(ws[0].clone())
    outs = [mx.mx_quantize_fp8(w, 32, "e8m0") for w in ws]
    yq = [torch.empty((C2_ROWS, C2_K), dtype=bf, device=dev) for _ in range(3)]
    qb = 2 * n + n + n // 32
    for kind, fn in (("quantize", lambda i: mx.mx_quantize_fp8(ws[i], 32, "e8m0", codes=outs[i][0], scales=outs[i][1])),
                     ("dequantize", lambda i: mx.mx_dequantize_fp8(outs[i][0], outs[i][1], 32, "e8m0", y=yq[i]))):
        for i in range(3):
            fn(i)
        evs = []
        for r in range(9):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn(r % 3)
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) for a, b in evs)[4]
        gbs = qb / (t * 1e-3) / 1e9
        res[f"{kind}_fp8.B32.e8m0.n{C2_ROWS}.k{C2_K}"] = {"us": round(t * 1e3, 2), "GB/s": round(gbs, 1),
                                                         "frac_hbm": round(gbs * 1e9 / PEAK_HBM, 3)}
    del ws, outs, yq

    for nn, copies in ((4096, 64), (14336, 20)):
        w = dev_bf16(synth.c3_weight(nn))
        c0, s0 = mx.mx_quantize_fp8(w, 32, "e8m0")
        del w
        cs = [(c0.clone(), s0.clone()) for _ in range(copies)]
        for m in (1, 16):
            x = dev_bf16(synth.c3_x(m))
            y = torch.empty((m, nn), dtype=bf, device=dev)

            def decode_step():
                sp = torch.cuda.current_stream().cuda_stream
                for c, sc in cs:
                    st = L.mx_gemm_fp8(x.data_ptr(), m, nn, 4096, 4096, c.data_ptr(), sc.data_ptr(), 32,
                                       mx.FMT["e8m0"], 1.0, y.data_ptr(), 1, nn, sp)
                    if st:
                        raise mx.MXError(st, "mx_gemm_fp8")

            side = torch.cuda.Stream()
            with torch.cuda.stream(side):
                decode_step()
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                decode_step()
            graph.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(5):
                graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            tot = e0.elapsed_time(e1) / 5
            byt = nn * 4096 + nn * 4096 // 32 + m * 4096 * 2 + m * nn * 2
            gbs = byt * copies / (tot * 1e-3) / 1e9
            res[f"gemv_w8.m{m}.n{nn}.k4096"] = {
                "GB/s": round(gbs, 1), "frac_hbm": round(gbs * 1e9 / PEAK_HBM, 3),
                "us_per_launch": round(tot * 1e3 / copies, 2),
                "launches": f"{copies} distinct weights back to back (graph replay)"}
            del graph
        del cs, c0, s0

    w = dev_bf16(synth.c4_weight())
    c8, s8 = mx.mx_quantize_fp8(w, 32, "e8m0")
    del w
    x = dev_bf16(synth.c4_x())
    M, N, K = 2048, 28672, 8192
    y = torch.empty((M, N), dtype=bf, device=dev)
    fn = lambda: mx.mx_gemm_fp8(x, c8, s8, 32, "e8m0", y=y)
    time_launches(torch, stream, [fn], reps=1)
    ts = time_launches(torch, stream, [fn], reps=3)
    t = sorted(ts)[1]
    tf = 2 * M * N * K / (t * 1e-3) / 1e12
    res[f"gemm_w8.m{M}.n{N}.k{K}"] = {"TFLOP/s": round(tf, 1), "frac_peak_bf16": round(tf * 1e12 / PEAK_BF16, 4),
                                      "ms": round(t, 3)}
    log("fp8 fallback: " + ", ".join(f"{k} {v.get('GB/s', v.get('TFLOP/s'))}" for k, v in res.items()))
    return res


def measure_block_policy(mx, torch, inputs, error_split, dev, stream):
    """The sigma-driven block size on the sweep tensors: the standard deviation measured on the
    device (mx_tensor_stats, two fp64 passes; timed), the block size the policy picks from it,
    and that block's total MSE next to block 32's and the sweep's best, per scale format (the
    MSEs are the device error split's)."""
    n = C2_ROWS * C2_K
    out = torch.zeros(4, dtype=torch.float64, device=dev)
    work = torch.empty(mx.mx_tensor_stats_workspace_size(C2_ROWS, C2_K), dtype=torch.uint8, device=dev)
    per = error_split["per_config"]
    res = {}
    times = []
    for si, sigma in enumerate(SIGMAS):
        x = inputs[2 * si]
        mx.mx_tensor_stats(x, out=out, workspace=work, stream=stream)  # warm-up
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        st = mx.mx_tensor_stats(x, out=out, workspace=work, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
        mean, std, amax = (float(v) for v in st.cpu().numpy())
        b = mx.mx_adaptive_block_size(std)
        ent = {"std": std, "mean": mean, "absmax": amax, "policy_block": b}
        for f in FMTS:
            tot = {bb: per[f"s{sigma}.B{bb}.{f}"]["mse_total"] for bb in BLOCKS}
            best = min(tot, key=tot.get)
            ent[f] = {"mse_policy": tot[b], "mse_b32": tot[32], "best_block": best, "mse_best": tot[best]}
        res[f"s{sigma}"] = ent
    t = sorted(times)[len(times) // 2]
    res["stats_kernel"] = {"us": round(t * 1e3, 2), "bytes": 2 * 2 * n,
                           "GB/s": round(4 * n / (t * 1e-3) / 1e9, 1)}
    res["layer_blocks"] = {k: mx.mx_layer_block_size(k) for k in ("qkv", "ffn_gate_up", "output")}
    log(f"block policy: " + ", ".join(f"s{sg}: std {res[f's{sg}']['std']:.4f} -> B{res[f's{sg}']['policy_block']}"
                                       for sg in SIGMAS) + f"; stats {t * 1e3:.1f} us")
    return res


COPY_BYTES = 256 << 20  # calibration copy: 256 MiB read + 256 MiB written per launch


def pmc_run(mx, torch, np, synth, dev):
    """Five launches of the dominant kernel (block-32 E8M0 quantize of the sigma = 0.02
    weight) and five plain copies of COPY_BYTES, for the HBM byte counters."""
    w = synth.c2_weight(0.02)
    x = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).to(dev)
    codes = torch.empty((C2_ROWS, C2_K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((C2_ROWS, C2_K // 32), dtype=torch.uint8, device=dev)
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    for _ in range(5):
        flush.fill_(1)  # evict the previous launch's data from the Infinity Cache
        mx.mx_quantize(x, 32, "e8m0", codes=codes, scales=scales)
    for _ in range(5):
        flush.fill_(1)
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"pmc run: 5 x quantize ({quant_bytes(C2_ROWS * C2_K, 32)} algorithmic bytes), "
        f"5 x copy ({COPY_BYTES} bytes read, {COPY_BYTES} written)")


def pmc_rows(mx, torch, np, synth, dev):
    """Three launches each of the decode GEMV (m 1, 4 and 16, n 14336, k 4096, block 32 E8M0), the
    405B-FFN GEMV (m 1, UE5M3 with a tensor scale), the 70B-FFN prefill GEMM in W4A16 and in
    W4A4 with tiled weight scales (its activation pre-pass is a quantize launch of its own),
    each after a 512 MB fill that evicts the Infinity Cache, then five copies of COPY_BYTES."""
    bf = torch.bfloat16

    def dev_bf16(a):
        return torch.from_numpy(a.view(np.int16)).view(bf).to(dev)

    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def launch3(what, fn):
        for _ in range(3):
            flush.fill_(1)
            fn()
        torch.cuda.synchronize()
        log(f"pmc rows: 3 x {what}")

    w = dev_bf16(synth.c3_weight(14336))
    c3, s3 = mx.mx_quantize(w, 32, "e8m0")
    del w
    x = dev_bf16(synth.c3_x(1))
    y = torch.empty((1, 14336), dtype=bf, device=dev)
    launch3(f"decode GEMV m 1 n 14336 k 4096 ({gemv_bytes(1, 14336, 4096, 32)} algorithmic bytes)",
            lambda: mx.mx_gemm(x, c3, s3, 32, "e8m0", 1.0, "a16", y=y))
    for m in (4, 16):
        xm = dev_bf16(synth.c3_x(m))
        ym = torch.empty((m, 14336), dtype=bf, device=dev)
        launch3(f"decode GEMV m {m} n 14336 k 4096 ({gemv_bytes(m, 14336, 4096, 32)} algorithmic bytes)",
                lambda: mx.mx_gemm(xm, c3, s3, 32, "e8m0", 1.0, "a16", y=ym))
    del c3, s3, x, y, xm, ym

    wh = synth.c5_weight()
    g = synth.c5_tensor_scale(wh)
    w = dev_bf16(wh)
    del wh
    N, K = 53248, 16384
    c5, s5 = mx.mx_quantize(w, 32, "ue5m3", g)
    del w
    torch.cuda.empty_cache()
    x = dev_bf16(synth.c5_x(1))
    y = torch.empty((1, N), dtype=bf, device=dev)
    launch3(f"405B-FFN GEMV m 1 ({gemv_bytes(1, N, K, 32)} algorithmic bytes)",
            lambda: mx.mx_gemm(x, c5, s5, 32, "ue5m3", g, "a16", y=y))
    del c5, s5, x, y
    torch.cuda.empty_cache()

    w = dev_bf16(synth.c4_weight())
    c4, s4 = mx.mx_quantize(w, 32, "e8m0")
    _, s4t = mx.mx_quantize(w, 32, "e8m0", layout="tiled")
    del w
    x = dev_bf16(synth.c4_x())
    M, N, K = 2048, 28672, 8192
    y = torch.empty((M, N), dtype=bf, device=dev)
    ws = torch.empty(mx.mx_gemm_workspace_size(M, N, K, 32, "a4"), dtype=torch.uint8, device=dev)
    launch3(f"W4A16 GEMM {M} x {N} x {K} ({2 * M * N * K} flops)",
            lambda: mx.mx_gemm(x, c4, s4, 32, "e8m0", 1.0, "a16", y=y))
    launch3(f"W4A4 GEMM {M} x {N} x {K}, tiled weight scales ({2 * M * N * K} flops)",
            lambda: mx.mx_gemm(x, c4, s4t, 32, "e8m0", 1.0, "a4", y=y, workspace=ws, layout="tiled"))
    del c4, s4, s4t, x, y, ws
    torch.cuda.empty_cache()

    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        flush.fill_(1)
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"pmc rows: 5 x copy ({COPY_BYTES} bytes read, {COPY_BYTES} written)")


def pmc_c5(mx, torch, np, synth, dev):
    """Three launches each of the 405B-FFN W4A16 product (53248 x 16384 UE5M3 weight with its
    per-tensor scale) at m 256 and m 4096, each after a 512 MB fill that evicts the Infinity
    Cache, for the L2 / matrix-core / vector counters of the wide-tile kernel."""
    wh = synth.c5_weight()
    g = synth.c5_tensor_scale(wh)
    w = torch.from_numpy(wh.view(np.int16)).view(torch.bfloat16).to(dev)
    del wh
    N, K = 53248, 16384
    c5, s5 = mx.mx_quantize(w, 32, "ue5m3", g)
    del w
    torch.cuda.empty_cache()
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    for m in (256, 4096):
        x = torch.from_numpy(synth.c5_x(m).view(np.int16)).view(torch.bfloat16).to(dev)
        y = torch.empty((m, N), dtype=torch.bfloat16, device=dev)
        for _ in range(3):
            flush.fill_(1)
            mx.mx_gemm(x, c5, s5, 32, "ue5m3", g, "a16", y=y)
        torch.cuda.synchronize()
        log(f"pmc c5: 3 x W4A16 {m} x {N} x {K} ({2 * m * N * K} flops)")


def library_ref(mx, torch, np, synth, dev, stream):
    """The 70B-FFN prefill GEMM (2048 x 28672 x 8192) in this library's W4A16 and W4A4 modes
    beside the vendor library's kernels for the same product, for context: hipBLASLt's bf16
    GEMM on the bf16 weight (torch.nn.functional.linear) and its MXFP4 GEMM with E8M0 block
    scales on the same FP4 codes and scales (torch._scaled_mm on float4_e2m1fn_x2 operands;
    it takes pre-quantized activations, so the activation codes come from mx_quantize first,
    while this library's W4A4 time includes that pre-pass).  Each entry is timed over five
    back-to-back launches queued behind an untimed one, so that host-side call overhead does
    not reach the GPU's timeline."""
    bf = torch.bfloat16
    M, N, K = 2048, 28672, 8192
    flops = 2 * M * N * K

    def dev_bf16(a):
        return torch.from_numpy(a.view(np.int16)).view(bf).to(dev)

    fp4 = getattr(torch, "float4_e2m1fn_x2", None)
    e8 = getattr(torch, "float8_e8m0fnu", None)
    if fp4 is not None and e8 is not None:
        # the vendor MXFP4 GEMM once on throw-away operands of the same shape, before this
        # library's first launch
        try:
            za = torch.zeros((M, K // 2), dtype=torch.uint8, device=dev).view(fp4)
            zb = torch.zeros((N, K // 2), dtype=torch.uint8, device=dev).view(fp4)
            sa = torch.full((M, K // 32), 127, dtype=torch.uint8, device=dev).view(e8)
            sb = torch.full((N, K // 32), 127, dtype=torch.uint8, device=dev).view(e8)
            torch._scaled_mm(za, zb.t(), scale_a=sa, scale_b=sb, out_dtype=bf)
            torch.cuda.synchronize()
            del za, zb, sa, sb
        except RuntimeError as e:  # under rocprofv3 the first heuristic query can fail
            log(f"library MXFP4 GEMM warm-up call failed: {str(e)[:160]}")
    w = dev_bf16(synth.c4_weight())
    c4, s4 = mx.mx_quantize(w, 32, "e8m0")
    _, s4t = mx.mx_quantize(w, 32, "e8m0", layout="tiled")
    x = dev_bf16(synth.c4_x())
    xc, xs = mx.mx_quantize(x, 32, "e8m0")
    y = torch.empty((M, N), dtype=bf, device=dev)
    ws = torch.empty(mx.mx_gemm_workspace_size(M, N, K, 32, "a4"), dtype=torch.uint8, device=dev)
    entries = {
        "w4a16": lambda: mx.mx_gemm(x, c4, s4, 32, "e8m0", 1.0, "a16", y=y),
        "w4a4_tiled_scales": lambda: mx.mx_gemm(x, c4, s4t, 32, "e8m0", 1.0, "a4", y=y, workspace=ws,
                                                layout="tiled"),
        "hipblaslt_bf16": lambda: torch.nn.functional.linear(x, w),
    }
    agree = None
    if fp4 is not None and e8 is not None:
        xa, wb = xc.view(fp4), c4.view(fp4)
        sxa, swb = xs.view(e8), s4.view(e8)
        try:
            y_lib = torch._scaled_mm(xa, wb.t(), scale_a=sxa, scale_b=swb, out_dtype=bf)
            mx.mx_gemm(x, c4, s4t, 32, "e8m0", 1.0, "a4", y=y, workspace=ws, layout="tiled")
            d = (y_lib.float() - y.float()).abs().max().item()
            agree = {"max_abs_diff_vs_w4a4": d, "max_abs_w4a4": y.float().abs().max().item()}
            entries["hipblaslt_mxfp4"] = lambda: torch._scaled_mm(xa, wb.t(), scale_a=sxa, scale_b=swb,
                                                                  out_dtype=bf)
        except RuntimeError as e:
            log(f"library MXFP4 GEMM unavailable: {e}")
    out = {}
    for name, fn in entries.items():
        fn()
        torch.cuda.synchronize()
        res = []
        for _ in range(3):
            fn()  # untimed: occupies the GPU while the timed launches are queued
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(5):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            res.append(a.elapsed_time(b) / 5)
        t = sorted(res)[1]
        out[name] = {"ms": round(t, 4), "TFLOP/s": round(flops / (t * 1e-3) / 1e12, 1)}
        log(f"library ref {name}: {t:.4f} ms")
    print(json.dumps({"library_ref": out, "shape": [M, N, K], "mxfp4_agreement": agree}), flush=True)


def load_traffic(kernel: str):
    """Counter-derived HBM bytes per launch for `kernel` from profiles/traffic.json, or None
    if absent or measured on a different source than the current one."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))[kernel]
    except (KeyError, ValueError):
        return None
    src = os.path.join(ROOT, "microscaling_fp4_weight_amd", "csrc", rec["source"])
    dev_h = os.path.join(ROOT, "microscaling_fp4_weight_amd", "csrc", "mx_device.h")
    h = hashlib.sha256(open(src, "rb").read() + open(dev_h, "rb").read()).hexdigest()[:16]
    if h != rec.get("source_sha"):
        return None
    return rec["bytes_per_launch"]


def time_launches(torch, stream, launches, reps=1, batch=4):
    """Per-launch durations (ms) from HIP events on the launch stream: for each of `reps`
    rounds, each launch runs `batch` times back to back between one pair of events, and the
    round's time is divided by `batch`.  Back to back, the host's call overhead (argument
    checks, marshalling) overlaps the previous launch instead of showing as idle GPU time."""
    evs = []
    for _ in range(reps):
        for fn in launches:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(batch):
                fn()
            b.record(stream)
            evs.append((a, b))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) / batch for a, b in evs]


def measure_rows(mx, L, torch, np, synth, dev, stream):
    """The GEMV / GEMM / two-level rows of the hot path, each timed with HIP events."""
    rows = {}
    bf = torch.bfloat16

    def dev_bf16(a):
        return torch.from_numpy(a.view(np.int16)).view(bf).to(dev)

    # decode GEMV: distinct weight copies (>= 512 MB) launched back to back, as a decode step
    # across layers would.  The launches are captured once in a HIP graph and replayed, so that
    # the GPU sees them back to back (from Python, each call's host overhead exceeds a small
    # GEMV's duration).
    for nn, copies in ((4096, 64), (14336, 20)):
        w = dev_bf16(synth.c3_weight(nn))
        c0, s0 = mx.mx_quantize(w, 32, "e8m0")
        _, s0p = mx.mx_quantize(w, 32, "e8m0", layout="preshuffled")  # same codes
        del w
        cs = [(c0.clone(), s0.clone(), s0p.clone()) for _ in range(copies)]
        for m, lay in ((1, 0), (1, 2), (4, 0), (16, 0)):
            x = dev_bf16(synth.c3_x(m))
            y = torch.empty((m, nn), dtype=bf, device=dev)

            def decode_step():
                sp = torch.cuda.current_stream().cuda_stream
                for c, s, sps in cs:
                    st = L.mx_gemm(x.data_ptr(), m, nn, 4096, 4096, c.data_ptr(),
                                   (sps if lay == 2 else s).data_ptr(), 32, mx.FMT["e8m0"], 1.0, lay, 0,
                                   y.data_ptr(), 1, nn, None, 0, sp)
                    if st:
                        raise mx.MXError(st, "mx_gemm")

            side = torch.cuda.Stream()
            with torch.cuda.stream(side):
                decode_step()  # eager warm-up
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                decode_step()
            graph.replay()
            torch.cuda.synchronize()
            reps = 5
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                graph.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            tot = e0.elapsed_time(e1) / reps  # ms per decode step (copies launches)
            byt = gemv_bytes(m, nn, 4096, 32)
            gbs = byt * copies / (tot * 1e-3) / 1e9
            rows[f"gemv_a16.m{m}.n{nn}.k4096" + (".preshuffled_scales" if lay == 2 else "")] = {
                "GB/s": round(gbs, 1), "frac_hbm": round(gbs * 1e9 / PEAK_HBM, 3),
                "us_per_launch": round(tot * 1e3 / copies, 2),
                "TFLOP/s": round(2 * m * nn * 4096 * copies / (tot * 1e-3) / 1e12, 2),
                "launches": f"{copies} distinct weights back to back (graph replay)"}
            del graph
        del cs, c0, s0, s0p
        log(f"decode GEMV n={nn} done")

    # 70B-FFN prefill: W4A16 and W4A4
    w = dev_bf16(synth.c4_weight())
    c4, s4 = mx.mx_quantize(w, 32, "e8m0")
    _, s4t = mx.mx_quantize(w, 32, "e8m0", layout="tiled")  # same codes, tiled scale order
    del w
    x = dev_bf16(synth.c4_x())
    M, N, K = 2048, 28672, 8192
    flops = 2 * M * N * K
    y = torch.empty((M, N), dtype=bf, device=dev)
    ws = torch.empty(mx.mx_gemm_workspace_size(M, N, K, 32, "a4"), dtype=torch.uint8, device=dev)
    for mode, layout, peak in (("a16", "rowmajor", PEAK_BF16), ("a4", "rowmajor", PEAK_FP4),
                               ("a4", "tiled", PEAK_FP4)):
        sc = s4t if layout == "tiled" else s4
        fn = lambda: mx.mx_gemm(x, c4, sc, 32, "e8m0", 1.0, mode, y=y, workspace=ws, layout=layout)
        time_launches(torch, stream, [fn], reps=2)
        ts = time_launches(torch, stream, [fn], reps=5)
        t = sorted(ts)[len(ts) // 2]
        tf = flops / (t * 1e-3) / 1e12
        key = f"gemm_{mode}.m{M}.n{N}.k{K}" + (".tiled_scales" if layout == "tiled" else "")
        rows[key] = {"TFLOP/s": round(tf, 1), "frac_peak": round(tf * 1e12 / peak, 4),
                     "peak_TFLOP/s": peak / 1e12, "ms": round(t, 3),
                     "includes": "activation pre-pass" if mode == "a4" else "-"}
        log(f"C4 {mode} {layout}: {t:.3f} ms, {tf:.0f} TFLOP/s")
    del c4, s4, s4t, x, y, ws
    torch.cuda.empty_cache()

    # 405B-FFN: offline two-level quantize, GEMV M=1, GEMM M=256 / 4096
    wh = synth.c5_weight()
    g = synth.c5_tensor_scale(wh)
    rows["c5_tensor_scale"] = g
    w = dev_bf16(wh)
    del wh
    N, K = 53248, 16384
    c5 = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    s5 = torch.empty((N, K // 32), dtype=torch.uint8, device=dev)
    fn = lambda: mx.mx_quantize(w, 32, "ue5m3", g, codes=c5, scales=s5)
    time_launches(torch, stream, [fn])
    ts = time_launches(torch, stream, [fn], reps=3)
    t = sorted(ts)[1]
    gbs = quant_bytes(N * K, 32) / (t * 1e-3) / 1e9
    rows["quantize.ue5m3.g.n53248.k16384"] = {"GB/s": round(gbs, 1),
                                              "frac_hbm": round(gbs * 1e9 / PEAK_HBM, 3),
                                              "ms": round(t, 3)}
    c5p, s5p = mx.mx_quantize(w, 32, "ue5m3", g, layout="preshuffled")  # same codes as c5
    del w, c5p
    torch.cuda.empty_cache()
    x = dev_bf16(synth.c5_x(1))
    y = torch.empty((1, N), dtype=bf, device=dev)
    fn = lambda: mx.mx_gemm(x, c5, s5p, 32, "ue5m3", g, "a16", y=y, layout="preshuffled")
    time_launches(torch, stream, [fn])
    ts = time_launches(torch, stream, [fn], reps=3)
    t = sorted(ts)[1]
    gbs = gemv_bytes(1, N, K, 32) / (t * 1e-3) / 1e9
    rows[f"gemm_a16.ue5m3.g.m1.n{N}.k{K}.preshuffled_scales"] = {
        "TFLOP/s": round(2 * N * K / (t * 1e-3) / 1e12, 2), "ms": round(t, 3), "GB/s": round(gbs, 1),
        "frac_hbm": round(gbs * 1e9 / PEAK_HBM, 3)}
    del x, y, s5p
    for m in (1, 256, 4096):
        x = dev_bf16(synth.c5_x(m))
        y = torch.empty((m, N), dtype=bf, device=dev)
        fn = lambda: mx.mx_gemm(x, c5, s5, 32, "ue5m3", g, "a16", y=y)
        time_launches(torch, stream, [fn])
        ts = time_launches(torch, stream, [fn], reps=3)
        t = sorted(ts)[1]
        tf = 2 * m * N * K / (t * 1e-3) / 1e12
        ent = {"TFLOP/s": round(tf, 2), "ms": round(t, 3)}
        if m == 1:
            gbs = gemv_bytes(1, N, K, 32) / (t * 1e-3) / 1e9
            ent.update({"GB/s": round(gbs, 1), "frac_hbm": round(gbs * 1e9 / PEAK_HBM, 3)})
        else:
            ent.update({"frac_peak_bf16": round(tf * 1e12 / PEAK_BF16, 4)})
        rows[f"gemm_a16.ue5m3.g.m{m}.n{N}.k{K}"] = ent
        log(f"C5 m={m}: {t:.3f} ms")
        del x, y
    del c5, s5
    torch.cuda.empty_cache()
    return rows


def host_info():
    """Host cores and CPU model, as the process sees them."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_count": os.cpu_count(), "usable_cpus": len(os.sched_getaffinity(0)), "model": model}


# GEMM rows the oracle is timed on: (row name, full m, n, k, sampled rows, sampled columns, mode)
ORACLE_GEMM = (
    ("gemv_a16.m1.n14336.k4096", 1, 14336, 4096, 1, 14336, "a16"),
    ("gemv_a16.m16.n14336.k4096", 16, 14336, 4096, 16, 14336, "a16"),
    ("gemm_a16.m2048.n28672.k8192", 2048, 28672, 8192, 16, 4096, "a16"),
    ("gemm_a4.m2048.n28672.k8192", 2048, 28672, 8192, 16, 4096, "a4"),
    ("gemm_a16.ue5m3.g.m4096.n53248.k16384", 4096, 53248, 16384, 16, 2048, "a16"),
)


def cpu_baseline(np, synth, gpu_value, rows):
    """The CPU oracle as it stands (single-threaded C, fp64 where it computes in floating
    point), on the host's first usable core, on bounded samples of the workloads:
     * the step's workload (`value`): quantize + dequantize of the first 384 of 4096 rows of
       each sigma's Llama-7B FFN weight, every block size and scale format (GB/s of the same
       algorithmic bytes as the GPU step);
     * the GEMM oracle (dequantize, then an fp64 product): the decode GEMV rows in full (one
       and sixteen activation rows, 14336 x 4096 weight), and 16 activation rows against a
       slice of weight rows for the 70B-FFN prefill (W4A16 and W4A4) and the 405B-FFN m = 4096
       product; their full-size times are estimated from a 16-row and a 1-row run of the same
       weight slice (per weight row: one dequantization plus one dot product per activation
       row), scaled to all n rows;
     * the tiny round trip in full (256 x 256 fp32 weight, block 32 E4M3: quantize, dequantize,
       GEMV) and the 405B-FFN weight's offline quantize (UE5M3 with its tensor scale) on its
       first 512 of 53248 rows, scaled to all rows.
    Inputs are generated and the sampled weights quantized before the clock starts; only the
    oracle calls are timed."""
    import oracle
    host = host_info()
    sample_rows = 384
    c2 = {sigma: synth.c2_weight(sigma, row0=0, nrows=sample_rows) for sigma in SIGMAS}
    gemm_inputs = []
    for name, m, n, k, ms, ns, mode in ORACLE_GEMM:
        if k == 4096:
            x, w, fmt, g = synth.c3_x(m), synth.c3_weight(n, row0=0, nrows=ns), "e8m0", 1.0
        elif k == 8192:
            x, w, fmt, g = synth.c4_x(row0=0, nrows=ms), synth.c4_weight(row0=0, nrows=ns), "e8m0", 1.0
        else:
            g = (rows or {}).get("c5_tensor_scale")
            if g is None:
                g = synth.c5_tensor_scale(synth.c5_weight())
            x, w, fmt = synth.c5_x(m, row0=0, nrows=ms), synth.c5_weight(row0=0, nrows=ns), "ue5m3"
        wc, wsc = oracle.quantize(w, 32, fmt, g)
        gemm_inputs.append((x[:ms], wc, wsc, fmt, g))
        del w
    c1w, c1x = synth.c1_weight(), synth.c1_x()
    c5_rows = 512
    c5g = (rows or {}).get("c5_tensor_scale")
    if c5g is None:
        c5g = synth.c5_tensor_scale(synth.c5_weight())
    c5w = synth.c5_weight(row0=0, nrows=c5_rows)
    cpu = sorted(os.sched_getaffinity(0))[0]
    saved = os.sched_getaffinity(0)
    os.sched_setaffinity(0, {cpu})
    try:
        t0 = time.perf_counter()
        byt = 0
        for sigma in SIGMAS:
            w = c2[sigma]
            for b in BLOCKS:
                for f in FMTS:
                    c, sc = oracle.quantize(w, b, f)
                    oracle.dequantize(c, sc, C2_K, b, f, 1.0, "bf16")
                    byt += 2 * quant_bytes(sample_rows * C2_K, b)
        dt = time.perf_counter() - t0
        gemm = {}
        for (name, m, n, k, ms, ns, mode), (x, wc, wsc, fmt, g) in zip(ORACLE_GEMM, gemm_inputs):
            t1 = time.perf_counter()
            oracle.gemm(x, wc, wsc, 32, fmt, g, mode)
            gt = time.perf_counter() - t1
            if (ms, ns) == (m, n):
                est = gt
            else:
                # the oracle dequantizes each weight row once and then runs one fp64 dot product
                # per activation row: time = (n / ns) (d + m c); a one-row run gives d + c
                t1 = time.perf_counter()
                oracle.gemm(x[:1], wc, wsc, 32, fmt, g, mode)
                g1 = time.perf_counter() - t1
                c = max(gt - g1, 0.0) / (ms - 1)
                est = (n / ns) * (g1 - c + m * c)
            ent = {"s": round(gt, 3), "GFLOP/s": round(2 * ms * ns * k / gt / 1e9, 3),
                   "full_s": round(est, 2), "sample": f"{ms}x{ns} of {m}x{n}"}
            g_row = (rows or {}).get(name)
            if g_row is not None:
                gpu_s = g_row["us_per_launch"] * 1e-6 if "us_per_launch" in g_row else g_row["ms"] * 1e-3
                ent["gpu_speedup"] = round(est / gpu_s, 1)
            gemm[name] = ent
        t1 = time.perf_counter()
        c, sc = oracle.quantize(c1w, 32, "e4m3")
        oracle.dequantize(c, sc, 256, 32, "e4m3")
        oracle.gemm(c1x, c, sc, 32, "e4m3", 1.0, "a16")
        gemm["c1_round_trip_and_gemv"] = {"s": round(time.perf_counter() - t1, 4), "sample": "in full"}
        t1 = time.perf_counter()
        oracle.quantize(c5w, 32, "ue5m3", c5g)
        qt = time.perf_counter() - t1
        ent = {"s": round(qt, 3), "full_s": round(qt * 53248 / c5_rows, 1), "sample": f"{c5_rows} of 53248 rows"}
        g_row = (rows or {}).get("quantize.ue5m3.g.n53248.k16384")
        if g_row is not None:
            ent["gpu_speedup"] = round(qt * 53248 / c5_rows / (g_row["ms"] * 1e-3), 1)
        gemm["quantize.ue5m3.g.n53248.k16384"] = ent
    finally:
        os.sched_setaffinity(0, saved)
    value = byt / dt / 1e9
    log(f"cpu oracle sample: {dt:.1f}s quantize+dequantize, "
        + ", ".join(f"{k} {v['s']}s" for k, v in gemm.items()))
    return {"value": round(value, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "seconds": round(dt, 2), "gpu_speedup": round(gpu_value / value, 1),
            "sample": f"first {sample_rows} of {C2_ROWS} rows of each sigma's 4096x11008 weight, all 63 "
                      "(sigma, block, format) quantize + dequantize; single-threaded C oracle pinned to one core",
            "host": host, "pinned_cpu": cpu, "gemm": gemm}


if __name__ == "__main__":
    main()
