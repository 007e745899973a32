"""Runs the oracle's per-(sequence, layer) decode on several host threads.

Test infrastructure, like the rest of this package: only tests/, the smoke
check and bench.py's CPU-baseline leg use it.  It holds none of the method's
arithmetic: every result comes from attention.decode_layer (or
kivi.decode_layer) called unchanged on one (sequence, layer) piece, and the
pieces' block masses are summed per sequence in layer order, as
attention.decode_step sums them.  NumPy releases the interpreter lock inside
its array loops and BLAS calls, so pieces on different threads run in
parallel; each thread's BLAS is limited so that threads x BLAS threads stays
within the cores given.
"""
from __future__ import annotations

import os
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import attention as OA
from . import kivi as KV


def host_threads(cap: int = 16) -> int:
    """CPUs this process may run on, at most `cap`."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:   # not Linux
        n = os.cpu_count() or 1
    return max(1, min(cap, n))


def decode_layers(q, host_layer, lens, layers, scale: float, kv_format: str = "fp16",
                  threads: int = None, blas_threads: int = 2, progress=None):
    """The decode of every (sequence, layer) piece, threads pieces at a time.

    q:           [B][L][64][D] queries (fp16 or wider).
    host_layer:  host_layer(s, layer) -> sequence s's blocks of that layer in
                 logical order, [nb][1][2][8][16][D] (fp16 values, or E4M3
                 codes); called on the worker threads.
    lens:        tokens per sequence; layers: the layers to decode.
    Returns (out [B][L][64][D] fp64, NaN outside `layers`; list of per-sequence
    block mass summed over `layers`; dict with the wall time, the summed time
    spent in host_layer and the thread counts).
    """
    from threadpoolctl import threadpool_limits

    q = np.asarray(q)
    B = q.shape[0]
    layers = list(layers)
    threads = host_threads() if threads is None else max(1, int(threads))
    blas_threads = max(1, int(blas_threads))
    workers = max(1, threads // blas_threads)
    out = np.full(q.shape, np.nan, dtype=np.float64)
    piece_mass = {}
    fetch_s = [0.0] * (B * len(layers))

    def piece(k):
        s, li = divmod(k, len(layers))
        layer = layers[li]
        t = time.perf_counter()
        blocks = host_layer(s, layer)
        fetch_s[k] = time.perf_counter() - t
        n = int(lens[s])
        tbl = np.arange(blocks.shape[0])
        if kv_format == "kivi2":
            o, ms = KV.decode_layer(q[s, layer], blocks, tbl, n, 0, scale)
        else:
            o, ms = OA.decode_layer(q[s, layer], blocks, tbl, n, 0, scale, kv_format)
        out[s, layer] = o
        piece_mass[k] = ms
        if progress is not None and li % 10 == 9:
            progress(f"oracle: sequence {s}, layer {layer} done")
        return k

    t0 = time.perf_counter()
    with threadpool_limits(limits=blas_threads):
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(piece, range(B * len(layers))))
    wall = time.perf_counter() - t0
    masses = []
    for s in range(B):
        mass = np.zeros(-(-int(lens[s]) // 16), dtype=np.float64)
        for li in range(len(layers)):
            mass += piece_mass[s * len(layers) + li]
        masses.append(mass)
    info = dict(wall_s=wall, fetch_s=float(sum(fetch_s)), workers=workers,
                blas_threads=blas_threads, threads=workers * blas_threads)
    return out, masses, info
