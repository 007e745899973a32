"""kvs_decode_step_noalloc against kvs_decode_step: the same kernels over the
library's own scratch instead of a caller workspace.

Both run the same split with the same kernels, so outputs and block masses
must agree bit for bit (a stronger bar than the oracle's tolerance).  The
calls run in a row on one GPU, a large one then smaller ones, so each call
finds the previous call's partials in the shared scratch: anything read
before it is written would show.  Calls go through the C ABI (ctypes).
"""
import numpy as np
import pytest
import torch

import workload as W
from paged_gqa_kv_amd import _abi, api
from paged_gqa_kv_amd.session import DecodeSession

from . import parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _case(msg):
    print(f"\n[case] {msg}", flush=True)


def _noalloc(sess, q, status, layer_begin=None, layer_end=None, accumulate=0):
    m = sess.m
    lb = sess.layer_begin if layer_begin is None else layer_begin
    le = sess.layer_end if layer_end is None else layer_end
    out = torch.full_like(sess.out, float("nan"))
    mass = torch.full_like(sess.mass, float("nan")) if not accumulate else sess.mass.clone()
    api.decode_step_noalloc(sess.shape, q, m.pool, m.pool_blocks, m.block_table, m.max_blocks,
                            m.seq_lens, m.meta_offsets, m.batch, m.total_blocks, lb, le,
                            api.DEFAULT_SCALE, out, mass, accumulate, sess.split_blocks, status)
    return out, mass


def _same(a, b, rows=None):
    x = a if rows is None else a[rows]
    y = b if rows is None else b[rows]
    assert torch.equal(x.view(torch.int16) if x.dtype == torch.float16 else x.view(torch.int32),
                       y.view(torch.int16) if y.dtype == torch.float16 else y.view(torch.int32))


def _compare(m, split_blocks=0, steps=(0,), layer_ranges=None):
    sess = DecodeSession(m, split_blocks=split_blocks)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    need = api.decode_workspace_bytes(sess.shape, m.batch, m.max_blocks, m.total_blocks, 0,
                                      m.num_layers, sess.split_blocks)
    print(f"  scratch needed {need} of {_abi.KVS_NOALLOC_SCRATCH_BYTES} bytes, split "
          f"{sess.split_blocks}", flush=True)
    for step in steps:
        q = W.make_query(m, step)
        if layer_ranges is None:
            sess.decode(q)
            out, mass = _noalloc(sess, q, status)
        else:   # per-layer-range calls, mass accumulated
            for k, (lb, le) in enumerate(layer_ranges):
                sess.decode(q, accumulate=int(k > 0), layer_begin=lb, layer_end=le)
            out = torch.full_like(sess.out, float("nan"))
            mass = torch.zeros_like(sess.mass)
            for k, (lb, le) in enumerate(layer_ranges):
                o, mass = _noalloc_into(sess, q, status, lb, le, mass, out, accumulate=int(k > 0))
        torch.cuda.synchronize()
        _same(out, sess.out)
        _same(mass[:m.total_blocks], sess.mass[:m.total_blocks])
    assert int(status.item()) == 0
    assert sess.status() == 0
    return sess, out, mass


def _noalloc_into(sess, q, status, lb, le, mass, out, accumulate):
    m = sess.m
    api.decode_step_noalloc(sess.shape, q, m.pool, m.pool_blocks, m.block_table, m.max_blocks,
                            m.seq_lens, m.meta_offsets, m.batch, m.total_blocks, lb, le,
                            api.DEFAULT_SCALE, out, mass, accumulate, sess.split_blocks, status)
    return out, mass


def test_noalloc_matches_the_workspace_entry_point_on_calls_in_a_row():
    _case("noalloc vs kvs_decode_step: 3 layers x ragged batch, then a smaller batch")
    big = W.materialise(W.custom("na-big", 3, [5000, 300, 77, 16 * 300 + 9], seed=41,
                                 spare_blocks=6), DEV)
    sess, out, mass = _compare(big, steps=(0, 1))
    h = P.host(big)
    out_ref, mass_ref = P.oracle_decode(h, W.make_query(big, 1))
    P.check_out(out, out_ref, range(3))
    P.check_mass(mass, mass_ref, big.meta_offsets.cpu().numpy())
    del sess

    _case("noalloc vs kvs_decode_step: second call, 1 layer x 2 short sequences")
    small = W.materialise(W.custom("na-small", 1, [100, 40], seed=42, spare_blocks=2), DEV)
    sess, out, mass = _compare(small, split_blocks=4)
    out_ref, mass_ref = P.oracle_decode(P.host(small), W.make_query(small, 0))
    P.check_out(out, out_ref, range(1))
    P.check_mass(mass, mass_ref, small.meta_offsets.cpu().numpy())


def test_noalloc_128k_context_in_layer_ranges():
    """The 128K-token sequence at 8 layers, decoded in two layer ranges with the
    block mass accumulated, then a smaller call."""
    _case("noalloc vs kvs_decode_step: 131,072 tokens x 8 layers in two ranges of 4")
    m = W.materialise(W.custom("na-128k", 8, [131072], seed=43, spare_blocks=4), DEV)
    _compare(m, layer_ranges=[(0, 4), (4, 8)])
    del m
    torch.cuda.empty_cache()
    _case("noalloc vs kvs_decode_step: then 2 layers x 3 sequences")
    m2 = W.materialise(W.custom("na-after", 2, [1024, 33, 500], seed=44, spare_blocks=3), DEV)
    _compare(m2)


def test_noalloc_status_word_and_oversize_rejection():
    _case("noalloc: device-data error lands in the caller's status word; oversize call rejected")
    m = W.materialise(W.custom("na-status", 1, [64, 64], seed=45, spare_blocks=2), DEV)
    sess = DecodeSession(m)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    bad = m.block_table.clone()
    bad[1, 2] = m.pool_blocks + 5          # a physical id outside the pool
    out = torch.zeros_like(sess.out)
    mass = torch.zeros_like(sess.mass)
    api.decode_step_noalloc(sess.shape, W.make_query(m, 0), m.pool, m.pool_blocks, bad,
                            m.max_blocks, m.seq_lens, m.meta_offsets, m.batch, m.total_blocks,
                            0, 1, api.DEFAULT_SCALE, out, mass, 0, sess.split_blocks, status)
    torch.cuda.synchronize()
    assert int(status.item()) & _abi.KVS_DEV_BAD_BLOCK_ID
    assert np.isfinite(out.float().cpu().numpy()).all()
    with pytest.raises(api.KvsError) as e:
        api.decode_step_noalloc(api.shape(80), W.make_query(m, 0), m.pool, m.pool_blocks,
                                m.block_table, 8192, m.seq_lens, m.meta_offsets, 1, 8192, 0, 80,
                                api.DEFAULT_SCALE, out, mass, 0, 0, status)
    assert e.value.code == _abi.KVS_E_WORKSPACE
