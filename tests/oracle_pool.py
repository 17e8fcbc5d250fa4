"""The CPU oracle fanned out over host processes for the full-size parity tests.

Each worker regenerates its own slice of weight rows from the seeded generator (so no large
array crosses a process boundary on the way in), quantizes it with the oracle and runs the
oracle's fp64 product for the requested activation rows.  Workers never touch the GPU; they
are started with the spawn method, so the parent's GPU state is not inherited.
"""
from __future__ import annotations

import concurrent.futures
import multiprocessing
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402


def _weight(name: str, row0: int, nrows: int):
    import synth
    if name == "c3.4096":
        return synth.c3_weight(4096, row0=row0, nrows=nrows)
    if name == "c3.14336":
        return synth.c3_weight(14336, row0=row0, nrows=nrows)
    if name == "c4":
        return synth.c4_weight(row0=row0, nrows=nrows)
    if name == "c5":
        return synth.c5_weight(row0=row0, nrows=nrows)
    raise KeyError(name)


def _activations(name: str, m: int, rows):
    import synth
    if name.startswith("c3"):
        return synth.c3_x(m)[rows]
    if name == "c4":
        return np.concatenate([synth.c4_x(row0=int(r), nrows=1) for r in rows])
    return np.concatenate([synth.c5_x(m, row0=int(r), nrows=1) for r in rows])


def _slice_job(name, row0, nrows, fmt, g, gemms):
    """Quantize weight rows [row0, row0 + nrows) with the oracle, and for each (m, rows, mode)
    in gemms return the fp64 product and sum |x w| over those weight rows."""
    import oracle
    w = _weight(name, row0, nrows)
    c, s = oracle.quantize(w, 32, fmt, g)
    del w
    outs = []
    for m, rows, mode in gemms:
        x = _activations(name, m, rows)
        outs.append(oracle.gemm(x, c, s, 32, fmt, g, mode))
    return row0, c, s, outs


def workers() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


def full_weight(name: str, n: int, fmt: str, g: float, gemms, pieces: int | None = None):
    """Oracle codes and scales of the whole n-row weight `name`, and for every (m, rows, mode)
    in gemms the fp64 product Y and A = sum |x w| over all n weight rows (Y, A: len(rows) x n)."""
    pieces = pieces or 4 * workers()
    step = -(-n // pieces)
    codes = scales = None
    ys = [None] * len(gemms)
    ctx = multiprocessing.get_context("spawn")
    with concurrent.futures.ProcessPoolExecutor(max_workers=workers(), mp_context=ctx) as ex:
        futs = [ex.submit(_slice_job, name, r0, min(step, n - r0), fmt, g, gemms) for r0 in range(0, n, step)]
        for f in concurrent.futures.as_completed(futs):
            r0, c, s, outs = f.result()
            if codes is None:
                codes = np.empty((n, c.shape[1]), dtype=np.uint8)
                scales = np.empty((n, s.shape[1]), dtype=np.uint8)
            codes[r0:r0 + c.shape[0]] = c
            scales[r0:r0 + s.shape[0]] = s
            for i, (y, a) in enumerate(outs):
                if ys[i] is None:
                    ys[i] = (np.empty((y.shape[0], n)), np.empty((y.shape[0], n)))
                ys[i][0][:, r0:r0 + y.shape[1]] = y
                ys[i][1][:, r0:r0 + y.shape[1]] = a
    return codes, scales, ys
