"""GPU: the decode-timing hook (kvs_set_decode_events).  With events set, each
decode form (fp16 with one or two KV heads per wave, E4M3, KIVI, paired fp16 and E4M3)
records them around its decode kernel; the results are the bits of an untimed
call, the timed interval lies inside the call's wall time, and turning the hook
off leaves the events alone.  Both the default events and events without the
system-scope fence (as the bench creates them) are covered."""
import ctypes
import time

import numpy as np
import pytest
import torch

import workload as W
from paged_gqa_kv_amd import api
from paged_gqa_kv_amd.session import DecodeSession, pair_plan

pytestmark = pytest.mark.gpu

DEV = "cuda"
DISABLE_SYSTEM_FENCE = 0x20000000


def _case(msg):
    print(f"\n[case] {msg}", flush=True)


def _bits(t):
    return t.contiguous().view(torch.int16 if t.dtype == torch.float16 else torch.int32)


class _Events:
    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, flags):
        ev = ctypes.c_void_p()
        assert self.hip.hipEventCreateWithFlags(ctypes.byref(ev), flags) == 0
        return ev.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a),
                                            ctypes.c_void_p(b)) == 0
        return float(ms.value)

    def destroy(self, ev):
        self.hip.hipEventDestroy(ctypes.c_void_p(ev))


def _workload(kind):
    if kind in ("fp16-one-head", "e4m3", "kivi2", "fp16-paired", "e4m3-paired"):
        lens = [700, 100, 333, 288, 1000, 40, 517]
        wl = W.custom("timing", 2, lens, seed=31, spare_blocks=8,
                      shared_prefix_tokens=288 if kind.endswith("paired") else 0)
    else:   # sequences that fill their splits: one wave serves two KV heads
        wl = W.custom("timing2", 2, [1024, 1024], seed=32, spare_blocks=4)
    if kind.startswith("e4m3"):
        wl = W.as_e4m3(wl)
    elif kind == "kivi2":
        wl = W.as_kivi2(wl)
    return W.materialise(wl, DEV)


def _session(m, kind, split):
    if kind.endswith("paired"):
        return DecodeSession(m, split_blocks=split, pair_role=pair_plan(m.table_host, m.blocks))
    return DecodeSession(m, split_blocks=split)


@pytest.mark.parametrize("flags", [0, DISABLE_SYSTEM_FENCE])
@pytest.mark.parametrize("kind,split", [("fp16-one-head", 8), ("fp16-two-heads", 16),
                                        ("e4m3", 8), ("kivi2", 16), ("fp16-paired", 8),
                                        ("e4m3-paired", 8)])
def test_timed_decode_gives_untimed_bits(kind, split, flags):
    _case(f"{kind} split_blocks={split}, decode with and without timing events, flags={flags:#x}")
    m = _workload(kind)
    plain = _session(m, kind, split)
    timed = _session(m, kind, split)
    ev = _Events()
    before, after = ev.create(flags), ev.create(flags)
    try:
        for step in range(2):
            q = W.make_query(m, step)
            plain.decode(q)
            torch.cuda.synchronize()
            api.set_decode_events(before, after)
            try:
                t0 = time.perf_counter()
                timed.decode(q)
                torch.cuda.synchronize()
                wall_ms = (time.perf_counter() - t0) * 1e3
            finally:
                api.set_decode_events(None, None)
            assert torch.equal(_bits(timed.out), _bits(plain.out)), step
            assert torch.equal(_bits(timed.mass), _bits(plain.mass)), step
            kern_ms = ev.elapsed_ms(before, after)
            assert 0.0 < kern_ms <= wall_ms, (kern_ms, wall_ms)
        assert plain.status() == 0 and timed.status() == 0
        # with the hook off again, no event is touched: a later decode leaves
        # the recorded interval as it was
        plain.decode(W.make_query(m, 5))
        torch.cuda.synchronize()
        assert ev.elapsed_ms(before, after) == kern_ms
    finally:
        ev.destroy(before)
        ev.destroy(after)


def test_decode_events_both_or_neither():
    with pytest.raises(Exception):
        api.set_decode_events(np.intp(1).item(), None)
    api.set_decode_events(None, None)
