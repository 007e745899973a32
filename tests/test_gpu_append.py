"""GPU parity of the KV append + block allocation step followed by decode and
scoring, against the oracle's append (oracle/paging.py), decode and scoring on
its own host copy of the cache."""
import numpy as np
import pytest
import torch

import workload as W
from oracle import paging as PG
from oracle import scoring as OS
from paged_gqa_kv_amd import api
from paged_gqa_kv_amd.session import DecodeSession

from . import parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _case(msg):
    print(f"\n[case] {msg}", flush=True)


def _rows(offsets, blocks):
    return np.concatenate([offsets[s] + np.arange(nb) for s, nb in enumerate(blocks)])


def _bits(x):
    return x.view(np.uint16) if x.dtype == np.float16 else x


@pytest.mark.parametrize("kv_format,split_blocks", [("fp16", 4), ("fp16", 0), ("e4m3", 4)])
def test_append_decode_score(kv_format, split_blocks):
    _case(f"append + decode + score for 40 steps, {kv_format} KV, split_blocks={split_blocks}")
    wl = W.custom("app", 2, [1, 15, 16, 31, 47, 300], seed=11, spare_blocks=30,
                  kv_format=kv_format)
    m = W.materialise(wl, DEV, extra_blocks=3)
    sess = DecodeSession(m, split_blocks=split_blocks)
    alpha = 0.15
    pol = OS.Policy(alpha=alpha)
    gpol = api.policy(alpha)
    offsets = m.meta_offsets.cpu().numpy()
    pool_h = m.pool.cpu().numpy().copy()
    table_h = m.table_host.astype(np.int64).copy()
    lens_h = np.array(m.lens, dtype=np.int64)
    free_h = m.free_stack.astype(np.int64).copy()
    top = int(free_h.size)
    state = OS.init_state(m.blocks, m.seq_ids.cpu().numpy())
    for step in range(40):
        k, v = W.new_token_kv(m, step)
        sess.append(k, v)
        top, allocs, rejected = PG.append_step(pool_h, table_h, lens_h, free_h, top,
                                               k.cpu().numpy(), v.cpu().numpy())
        assert rejected == []
        q = W.make_query(m, step)
        sess.decode(q)
        sess.score(step, gpol)
        torch.cuda.synchronize()
        # integer / byte state: bit-exact
        assert np.array_equal(m.seq_lens.cpu().numpy(), lens_h)
        assert int(sess.free_top.item()) == top
        blocks = [int(-(-n // 16)) for n in lens_h]
        tab = m.block_table.cpu().numpy()
        for s, nb in enumerate(blocks):
            assert np.array_equal(tab[s, :nb], table_h[s, :nb])
        if step % 13 == 0 or step == 39:
            live = np.unique(table_h[table_h >= 0])
            assert np.array_equal(_bits(m.pool[torch.from_numpy(live).to(DEV)].cpu().numpy()),
                                  _bits(pool_h[live]))
        # decode over the grown sequences
        h = dict(pool=pool_h, table=table_h, lens=list(lens_h), kv_format=kv_format)
        out_ref, mass_ref = P.oracle_decode(h, q)
        P.check_out(sess.out, out_ref, range(2))
        P.check_mass(sess.mass, mass_ref, offsets)
        # scoring with records created for new blocks
        state = OS.grow(state, blocks)
        state, stale = OS.score_update(state, mass_ref, step, pol)
        assert not stale.any()
        rec = sess.records()[_rows(offsets, blocks)]
        P.check_records(rec, state, pol)
    assert sess.status() == 0


def test_append_exhausts_the_free_stack():
    _case("append with too few free blocks: later sequences are not appended")
    wl = W.custom("exh", 1, [16, 32, 48, 5], seed=3, spare_blocks=2)
    m = W.materialise(wl, DEV, extra_blocks=2)
    sess = DecodeSession(m)
    lens_h = np.array(m.lens, dtype=np.int64)
    table_h = m.table_host.astype(np.int64).copy()
    pool_h = m.pool.cpu().numpy().copy()
    free_h = m.free_stack.astype(np.int64).copy()
    top = int(free_h.size)
    assert top == 2
    k, v = W.new_token_kv(m, 0)
    sess.append(k, v)
    top, allocs, rejected = PG.append_step(pool_h, table_h, lens_h, free_h, top,
                                           k.cpu().numpy(), v.cpu().numpy())
    torch.cuda.synchronize()
    assert rejected == [2]                   # sequences 0 and 1 took the two free blocks
    assert np.array_equal(m.seq_lens.cpu().numpy(), lens_h)
    assert int(sess.free_top.item()) == top == 0
    assert sess.status() & api._abi.KVS_DEV_POOL_EXHAUSTED


def test_append_batch_larger_than_one_work_group():
    """1,500 sequences: the allocation scan runs over two 1,024-sequence chunks
    and carries its count across them."""
    _case("append with batch 1500 (two allocation chunks), 1 layer, 18 steps")
    rng = np.random.default_rng(4)
    lens = [int(x) for x in rng.choice([15, 16, 17, 31, 32, 1], size=1500)]
    wl = W.custom("wide", 1, lens, seed=6, spare_blocks=1500 * 2 + 10)
    m = W.materialise(wl, DEV, extra_blocks=3)
    sess = DecodeSession(m)
    pool_h = m.pool.cpu().numpy().copy()
    table_h = m.table_host.astype(np.int64).copy()
    lens_h = np.array(m.lens, dtype=np.int64)
    free_h = m.free_stack.astype(np.int64).copy()
    top = int(free_h.size)
    for step in range(18):
        k, v = W.new_token_kv(m, step)
        sess.append(k, v)
        top, allocs, rejected = PG.append_step(pool_h, table_h, lens_h, free_h, top,
                                               k.cpu().numpy(), v.cpu().numpy())
        assert rejected == []
    torch.cuda.synchronize()
    assert np.array_equal(m.seq_lens.cpu().numpy(), lens_h)
    assert int(sess.free_top.item()) == top
    tab = m.block_table.cpu().numpy()
    for s, n in enumerate(lens_h):
        nb = -(-int(n) // 16)
        assert np.array_equal(tab[s, :nb], table_h[s, :nb]), s
    live = np.unique(table_h[table_h >= 0])
    assert np.array_equal(_bits(m.pool[torch.from_numpy(live).to(DEV)].cpu().numpy()),
                          _bits(pool_h[live]))
    assert sess.status() == 0
