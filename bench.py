#!/usr/bin/env python3
"""Benchmark of one paged GQA decode + block-scoring step on one MI355X.

A step is the whole hot path over one batch: paged decode attention with
per-block mass (kvs_decode_step), then the fused score update and
classification of every per-block record (kvs_score_update, classify=1).
Inputs (pool, tables, the step's queries) are resident in HBM before the
timed region starts.

Prints one JSON line:
  value          KV GB/s: logical K+V bytes one step reads / step time
  blocks_per_s   records scored per second
  roofline       the decode kernel alone, timed with HIP events recorded by
                 the library around its launch on the bench's stream; with
                 --pair-sharers its bytes are those the paired kernel loads
                 (a block two paired sequences share counted once)
  cpu_baseline   the fp64 oracle over one whole step of the same workload on
                 the host's cores (measured, with its thread counts)
  copy_probe     a 4 GiB device copy (read + write) and the library's
                 streaming read probe over a 16 GiB buffer, best of four grids;
                 frac_of_read_probe = roofline.achieved / that read rate
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E, published
READ_PROBE_GRIDS = (256, 512, 1024, 2048)   # work-groups swept by the streaming read probe
ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "paged_gqa_kv_amd", "csrc")
# Sources a decode kernel is compiled from; a committed counter summary is used
# only while their digest matches the one recorded with it.
KERNEL_SOURCES = {
    "paged_decode_gqa": ("kvs_decode.hip", "kvs_decode_tiles.h", "kvs_device.h",
                         "kvs_internal.h"),
    "paged_decode_pair": ("kvs_decode_paired.hip", "kvs_decode_tiles.h", "kvs_device.h",
                          "kvs_internal.h"),
    "paged_decode_kivi": ("kvs_kivi.hip", "kvs_device.h", "kvs_internal.h"),
}


def kernel_digest(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=16)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="decode-80L-128K")
    ap.add_argument("--kv-format", choices=("fp16", "e4m3", "kivi2"), default="fp16",
                    help="stored K/V format (e4m3: FP8 codes, half the bytes)")
    ap.add_argument("--alpha", type=float, default=None)
    ap.add_argument("--split-blocks", type=int, default=0)
    ap.add_argument("--append", action="store_true",
                    help="each step first appends one token per sequence (kvs_append_kv)")
    ap.add_argument("--pair-sharers", action="store_true",
                    help="fp16 / E4M3: pair sequences that share their first block "
                         "(kvs_decode_step_paired, kvs_decode_step_e4m3_paired), so a shared "
                         "block is loaded once per pair")
    ap.add_argument("--scrub-mib", type=int, default=0,
                    help="read a buffer of this many MiB before each timed step, outside the "
                         "step's timing, so a small workload cannot be served from the caches")
    ap.add_argument("--cpu-seconds", type=float, default=150.0,
                    help="cap on the oracle baseline's time: it stops after the layer chunk "
                         "that passes it (a whole 128K-token step takes well under it; "
                         "0 = skip)")
    ap.add_argument("--copy-probe-gib", type=float, default=4.0,
                    help="buffer size of the device copy probe (0 = skip)")
    ap.add_argument("--copy-probe-reps", type=int, default=20)
    ap.add_argument("--read-probe-gib", type=float, default=16.0,
                    help="buffer size of the streaming read probe run beside the copy probe")
    return ap.parse_args()


class HipEvents:
    """hipEvent_t handles from the HIP runtime already loaded by torch."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    # hipEventDisableSystemFence: these events only time the kernels and are read
    # after a full device synchronisation, so they need no system-scope fence,
    # which would add a cache write-back and invalidation at every record.
    DISABLE_SYSTEM_FENCE = 0x20000000

    def create(self):
        ev = ctypes.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(ctypes.byref(ev), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        return ev.value

    def record(self, ev, stream_handle: int):
        rc = self.hip.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream_handle))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def destroy(self, ev):
        self.hip.hipEventDestroy(ctypes.c_void_p(ev))


def _traffic(kernel: str, workload: str, split_blocks: int):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sha256") != kernel_digest(kernel) or rec.get("split_blocks") != split_blocks:
        return None
    return rec.get("hbm_bytes_per_launch")


def _copy_probe(gib: float, reps: int, read_gib: float):
    """Achievable streaming bandwidth: device-to-device copy of gib-GiB buffers,
    median of reps, counting bytes read plus bytes written (the method the
    Visual Reference's measurement box describes for its 87 %-of-spec figure).
    Beside it, the library's streaming read probe (kvs_stream_probe, mode 0)
    over a read_gib-GiB buffer at several grids, the best of them: the read-only
    rate a decode could at best reach."""
    import torch

    from paged_gqa_kv_amd import api

    n = int(gib * 2**30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    sink = torch.empty(1 << 20, dtype=torch.int32, device="cuda")

    def median_s(fn):
        fn()
        times = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            times.append(a.elapsed_time(b) / 1e3)
        times.sort()
        return times[len(times) // 2]

    med = median_s(lambda: dst.copy_(src))
    del src, dst
    nr = int(read_gib * 2**30) // 16 * 16
    rsrc = torch.empty(nr, dtype=torch.uint8, device="cuda")   # contents do not matter
    # 1 to 8 work-groups of 256 lanes per compute unit; the fastest counts
    by_grid = {g: median_s(lambda g=g: api.stream_probe(rsrc, sink, nr, 0, g))
               for g in READ_PROBE_GRIDS}
    grid = min(by_grid, key=by_grid.get)
    med_read = by_grid[grid]
    del rsrc, sink
    torch.cuda.empty_cache()
    return {"bytes_per_copy": 2 * n * 4, "median_s": med, "gbps": 2 * n * 4 / med / 1e9,
            "reps": reps, "read_probe_bytes": nr, "read_probe_median_s": med_read,
            "read_probe_gbps": nr / med_read / 1e9, "read_probe_grid": grid,
            "read_probe_gbps_by_grid": {str(g): round(nr / t / 1e9, 1) for g, t in by_grid.items()}}


def _cpu_baseline(m, alpha, budget_s):
    """The fp64 oracle (as it stands) over one whole decode step of the same
    workload (step 0's query, every layer and sequence), then the scoring of
    every record.  The oracle runs per (sequence, layer) on the host's cores
    (oracle/runner.py, up to 16 threads); layers are copied to host memory a
    chunk at a time before the chunk is timed, so the device-to-host copy is
    reported apart.  Stops after the chunk that passes budget_s of oracle time
    (a 128K-token step takes well under it)."""
    import numpy as np
    import torch

    import workload as W
    from oracle import runner as OR
    from oracle import scoring as OS

    q = W.make_query(m, 0).cpu().numpy()
    scale = 1.0 / math.sqrt(128.0)
    L = m.num_layers
    fmt = m.workload.kv_format
    threads = OR.host_threads(16)
    # one sequence: split each layer's BLAS over 2 threads; many: 1 thread per piece
    blas = 2 if m.batch == 1 else 1
    # pieces of 1M tokens hold 17 GB of fp64 keys and values each: fewer at a time
    if max(m.lens) > 262144:
        blas = 4
    chunk = max(1, threads // blas)
    copy_s = 0.0
    oracle_s = 0.0
    layers_done = 0
    masses = [np.zeros(nb) for nb in m.blocks]
    info = {}
    for l0 in range(0, L, chunk):
        layers = range(l0, min(L, l0 + chunk))
        tc = time.perf_counter()
        host = {}
        for layer in layers:   # device -> host copy of this chunk's blocks
            for s in range(m.batch):
                pids = torch.from_numpy(m.table_host[s, :m.blocks[s]].astype(np.int64)).to(
                    m.pool.device)
                host[s, layer] = m.pool[pids, layer].cpu().numpy()[:, None]
        copy_s += time.perf_counter() - tc
        _, ms, info = OR.decode_layers(q, lambda s, layer: host[s, layer], m.lens, layers, scale,
                                       kv_format=fmt, threads=threads, blas_threads=blas)
        oracle_s += info["wall_s"]
        for s in range(m.batch):
            masses[s] += ms[s]
        layers_done += len(layers)
        del host
        if oracle_s >= budget_s:
            break
    t = time.perf_counter()
    st = OS.init_state(m.blocks, list(range(m.batch)))
    OS.score_update(st, masses, 0, OS.Policy(alpha=alpha))
    oracle_s += time.perf_counter() - t
    if fmt == "kivi2":
        from oracle import kivi as KV
        per_layer = sum(8 * (KV.quant_boundary(n) // 16 * 2 * KV.TILE_BYTES +
                             (n - KV.quant_boundary(n)) * 128 * 2 * 2) for n in m.lens)
    else:
        per_layer = sum(m.lens) * 8 * 128 * 2 * (1 if fmt == "e4m3" else 2)
    kv_bytes = per_layer * layers_done
    try:
        from threadpoolctl import threadpool_info
        blas_lib = ", ".join(sorted({str(d.get("internal_api")) for d in threadpool_info()}))
    except Exception:  # reporting only
        blas_lib = "unknown"
    whole = layers_done == L
    return {
        "value": kv_bytes / oracle_s / 1e9,
        "unit": "GB/s",
        "cores": info.get("threads", threads),
        "threads": {"pieces_in_parallel": info.get("workers"), "blas_per_piece":
                    info.get("blas_threads"), "blas_library": blas_lib},
        "host_cpus": {"os_cpu_count": os.cpu_count(),
                      "affinity": len(os.sched_getaffinity(0))},
        "kind": "oracle",
        "blocks_scored_per_s": (m.total_blocks / oracle_s) if whole else None,
        "sample": (f"fp64 oracle decode of {'all' if whole else layers_done} of {L} layers "
                   f"for all {m.batch} sequence(s) of step 0 (measured, not extrapolated), "
                   f"plus scoring of all {m.total_blocks} records: {oracle_s:.1f} s of oracle "
                   f"time on {info.get('threads', threads)} threads, excluding {copy_s:.1f} s "
                   f"of device-to-host copy"),
        "seconds": oracle_s,
        "copy_seconds": copy_s,
        "whole_step": whole,
    }


def main():
    args = _parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this path shards by "
              "sequence or by block range across GPUs, which is not built here.", file=sys.stderr)
        sys.exit(2)
    if args.pair_sharers and (args.kv_format == "kivi2" or args.append):
        print("--pair-sharers runs the fp16 or E4M3 decode without appends", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import workload as W
    from paged_gqa_kv_amd import api
    from paged_gqa_kv_amd.session import DecodeSession

    if not torch.cuda.is_available():
        print("bench.py needs a GPU (torch.cuda.is_available() is False)", file=sys.stderr)
        sys.exit(1)
    wl = W.WORKLOADS[args.workload]
    if args.kv_format == "e4m3":
        wl = W.as_e4m3(wl)
    elif args.kv_format == "kivi2":
        wl = W.as_kivi2(wl)
    alpha = args.alpha if args.alpha is not None else wl.alphas[0]
    extra = 0
    if args.append:
        # room for the appended tokens: table entries, records and free pool blocks
        extra = (args.warmup + args.steps) // 16 + 2
        import dataclasses
        wl = dataclasses.replace(wl, spare_blocks=max(wl.spare_blocks, extra * wl.batch + 8))
    print(f"[bench] materialising {wl.name} on cuda:0", file=sys.stderr, flush=True)
    t0 = time.time()
    m = W.materialise(wl, "cuda", extra_blocks=extra)
    torch.cuda.synchronize()
    print(f"[bench] inputs ready in {time.time() - t0:.1f} s; pool {m.pool.numel() * 2 / 2**30:.2f} GiB",
          file=sys.stderr, flush=True)
    # quantised blocks for the pairs that leave the fp16 window during the run
    spare = 2 * m.batch * ((args.warmup + args.steps) // 32 + 2) if args.append else None
    sess = DecodeSession(m, split_blocks=args.split_blocks, kivi_spare_blocks=spare,
                         pair_role="auto" if args.pair_sharers else None)
    pol = api.policy(alpha)
    n_q = args.warmup + args.steps
    queries = [W.make_query(m, k) for k in range(n_q)]
    new_kv = [W.new_token_kv(m, k) for k in range(n_q)] if args.append else None

    def run_step(k, idx):
        """One step: [append], decode, score."""
        if new_kv is not None:
            sess.append(*new_kv[idx])
        sess.decode(queries[idx])
        sess.score(k, pol)
    torch.cuda.synchronize()

    ev = HipEvents()
    pairs = [(ev.create(), ev.create()) for _ in range(args.steps)]

    # warm-up on the same buffers; records are re-initialised afterwards so the
    # timed steps start from fresh records with steps 0..K-1
    for k in range(args.warmup):
        run_step(k, k)
    torch.cuda.synchronize()
    sess.reset_meta()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    lens_at_start = m.seq_lens.cpu().numpy().copy()
    # Inside the timed region the only markers are the two HIP events around
    # each decode kernel (the roofline's timing).  Each idles the queue for about
    # 4.5 us (8 x 8K tokens x 4 layers: a 173 us step without them, 182 us with
    # them, kernel trace), so per-step times come from those events and the
    # scoring kernels are timed apart afterwards.
    scrub = None
    bounds = ends = None
    if args.scrub_mib > 0:   # read between steps, outside each step's events
        scrub = torch.ones(args.scrub_mib << 18, dtype=torch.float32, device="cuda")
        bounds = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    end_hip = ev.create()
    start.record(stream)
    for k in range(args.steps):
        if scrub is not None:   # plain loads: evicts L2 and the Infinity Cache, leaves no dirty lines
            scrub.sum()
            bounds[k].record(stream)
        api.set_decode_events(*pairs[k])
        run_step(k, args.warmup + k)
        if scrub is not None:
            ends[k].record(stream)
    ev.record(end_hip, stream.cuda_stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    api.set_decode_events(None, None)
    decode_ms = [ev.elapsed_ms(a, b) for a, b in pairs]
    if scrub is None:
        total_ms = start.elapsed_time(end)
        # step k: from its decode kernel's start to the next one's (the last to the end)
        marks = [a for a, _ in pairs] + [end_hip]
        step_ms = sorted(ev.elapsed_ms(marks[k], marks[k + 1]) for k in range(args.steps))
    else:   # the steps alone: each from its first launch to its last
        step_ms = sorted(a.elapsed_time(b) for a, b in zip(bounds, ends))
        total_ms = sum(step_ms)
    ev.destroy(end_hip)
    del scrub
    for a, b in pairs:
        ev.destroy(a)
        ev.destroy(b)

    status = sess.status()
    if status:
        raise RuntimeError(f"device status bits set: {status:#x}")
    # sanity: every (layer, head) softmax sums to one, so each sequence's block
    # mass sums to layers x 64
    mass = sess.mass.cpu().numpy().astype(np.float64)
    offs = m.meta_offsets.cpu().numpy()
    lens_end = m.seq_lens.cpu().numpy()
    nb_end = (lens_end + 15) // 16
    nb_start = (lens_at_start + 15) // 16
    for s in range(m.batch):
        tot = mass[offs[s]:offs[s] + nb_end[s]].sum()
        if not math.isclose(tot, m.num_layers * 64, rel_tol=1e-4):
            raise RuntimeError(f"block mass of sequence {s} sums to {tot}")
    rec = sess.records()
    rows = np.concatenate([offs[s] + np.arange(nb_start[s]) for s in range(m.batch)])
    if (not (rec["touch_count"][rows] == args.steps).all()
            or not (rec["t_touch"][rows] == args.steps - 1).all()):
        raise RuntimeError("touch counts / timestamps do not match the steps run")
    if args.append and not np.array_equal(lens_end, lens_at_start + args.steps):
        raise RuntimeError("appends did not advance every sequence by one token per step")
    live = np.concatenate([offs[s] + np.arange(nb_end[s]) for s in range(m.batch)])
    rec = rec[live]

    # eviction candidates over the same records (the step after classification;
    # timed on its own, outside the step)
    ev_ms = []
    for _ in range(5):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        blk, _key = sess.evict_candidates(args.steps - 1, alpha)
        e1.record(stream)
        e1.synchronize()
        ev_ms.append(e0.elapsed_time(e1))
    ev_ms.sort()

    # the scoring kernels alone, timed apart on the same mass; the records the
    # run produced are put back afterwards
    saved_meta = sess.meta.clone()
    score_ms = []
    for rep in range(3):   # 8 back-to-back updates per sample, as they follow each other in a run
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(8):
            sess.score(args.steps + 8 * rep + i, pol)
        e1.record(stream)
        e1.synchronize()
        score_ms.append(e0.elapsed_time(e1) / 8)
    sess.meta.copy_(saved_meta)
    torch.cuda.synchronize()
    del saved_meta
    score_ms.sort()
    if int(blk.min().item()) < 0:
        raise RuntimeError("a sequence got no eviction candidate")

    kv_bytes = sess.kv_bytes_per_step
    fp16_bytes = sum(m.lens) * m.num_layers * 8 * 128 * 2 * 2
    if args.append:   # the average step reads the lengths in the middle of the run
        mean_tokens = float(lens_at_start.sum()) + m.batch * (args.steps + 1) / 2.0
        kv_bytes = int(mean_tokens * m.num_layers * 8 * 128 * 2 * sess.kv_elem_bytes)
        fp16_bytes = int(mean_tokens * m.num_layers * 8 * 128 * 2 * 2)
        if args.kv_format == "kivi2":   # stored bytes of each timed step's lengths
            per_step = []
            for k in range(args.steps):
                lens_k = lens_at_start + k + 1
                nq = np.array([api.kivi_quant_len(n) for n in lens_k])
                per_step.append(int((nq // 16 * 2 * 768 + (lens_k - nq) * 128 * 2 * 2).sum()))
            kv_bytes = int(sum(per_step) / len(per_step)) * m.num_layers * 8
    unique_bytes = m.unique_blocks * 16 * m.num_layers * 8 * 128 * 2 * sess.kv_elem_bytes
    if args.kv_format == "kivi2":
        resid = sum(m.lens) - int(sess.quant_lens_host.sum())
        unique_bytes = (sess.kivi_blocks * 2 * 768 + resid * 128 * 2 * 2) * m.num_layers * 8
    t_step = total_ms / 1e3 / args.steps
    value = kv_bytes / t_step / 1e9
    dec_avg = sum(decode_ms) / len(decode_ms) / 1e3
    # the roofline counts the bytes the kernel loads: under a pairing a shared
    # block once per pair, otherwise the logical bytes
    loaded_bytes = sess.kv_bytes_loaded_per_step if sess.pair_role is not None else kv_bytes
    achieved = loaded_bytes / dec_avg / 1e9
    if achieved > HBM_PEAK_GBPS and unique_bytes == loaded_bytes:
        raise RuntimeError(f"measured {achieved:.0f} GB/s exceeds the HBM peak: a timing bug")
    kernel = ("paged_decode_kivi" if args.kv_format == "kivi2" else
              "paged_decode_pair" if sess.pair_role is not None else "paged_decode_gqa")
    traffic = _traffic(kernel, wl.name, sess.split_blocks)
    tiers = np.bincount(rec["tier"], minlength=3)[:3].tolist()

    probe = None
    if args.copy_probe_gib > 0:
        print("[bench] copy probe", file=sys.stderr, flush=True)
        probe = _copy_probe(args.copy_probe_gib, args.copy_probe_reps, args.read_probe_gib)

    cpu = None
    if args.cpu_seconds > 0:
        print("[bench] timing the oracle baseline", file=sys.stderr, flush=True)
        cpu = _cpu_baseline(m, alpha, args.cpu_seconds)

    line = {
        "metric": "KV GB/s read + blocks scored/s per decode step; % of MI355X HBM peak",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp16": "fp16", "e4m3": "e4m3 KV, fp16 compute",
                  "kivi2": "2-bit KIVI KV + fp16 residual, fp16/fp32 compute"}[args.kv_format],
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "layers": m.num_layers,
            "batch": m.batch,
            "kv_format": args.kv_format,
            "append": bool(args.append),
            "context_tokens": int(sum(m.lens)),
            "records": m.total_blocks,
            "alpha": alpha,
            "split_blocks": sess.split_blocks,
            "kv_bytes_per_step": kv_bytes,
            "unique_kv_bytes_per_step": unique_bytes,
            "pair_sharers": bool(args.pair_sharers),
            "scrub_mib_between_steps": args.scrub_mib,
            "kv_bytes_loaded_per_step": loaded_bytes,
            "parallelism": "single GPU",
        },
        "blocks_scored_per_s": round(m.total_blocks / t_step, 1),
        "tokens_attended_per_s": round(sum(m.lens) * m.num_layers / t_step, 1),
        "fp16_equivalent_kv_gbps": round(fp16_bytes / t_step / 1e9, 2),
        "hbm_peak_frac": round(value / HBM_PEAK_GBPS, 4),
        "step_ms_median": round(step_ms[len(step_ms) // 2], 4),
        "step_ms_min": round(step_ms[0], 4),
        "score_update_us_median": round(score_ms[len(score_ms) // 2] * 1e3, 2),
        "records_scored_per_s_score_kernels": round(m.total_blocks / (score_ms[len(score_ms) // 2] / 1e3), 1),
        "decode_kernel_ms": round(dec_avg * 1e3, 4),
        "decode_share_of_step": round(dec_avg / t_step, 4),
        "tier_counts": tiers,
        "evict_candidates_us": round(ev_ms[len(ev_ms) // 2] * 1e3, 2),
        "host_wall_s": round(wall, 4),
        "copy_probe": probe,
        "frac_of_copy_probe": round(value / probe["gbps"], 4) if probe else None,
        "frac_of_read_probe": round(achieved / probe["read_probe_gbps"], 4) if probe else None,
        "roofline": {
            "bound": "hbm",
            "kernel": kernel,
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "traffic_source": (f"lookup of profiles/{kernel}_{wl.name}_traffic.json: "
                               "rocprofv3 FETCH_SIZE + WRITE_SIZE per launch, calibrated on a "
                               "copy kernel, keyed by the kernel's source digest and split"
                               if traffic is not None else
                               "no counter summary for the current kernel source and split"),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
