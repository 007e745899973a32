"""Pins for the oracle's KV append + block allocation."""
import numpy as np
import pytest

import workload as W
from oracle import attention as OA
from oracle import paging as PG
from oracle import scoring as OS


def _setup(lens, layers=2, spare=6, seed=1):
    wl = W.custom("app", layers, lens, seed=seed, spare_blocks=spare)
    m = W.materialise(wl, "cpu")
    pool = m.pool.numpy().copy()
    max_nb = max(m.blocks) + 3
    table = np.full((len(lens), max_nb), -1, dtype=np.int64)
    table[:, :m.table_host.shape[1]] = m.table_host
    used = set(int(x) for x in m.table_host[m.table_host >= 0].ravel())
    free = np.array([p for p in range(m.pool_blocks) if p not in used], dtype=np.int64)
    return m, pool, table, np.array(lens, dtype=np.int64), free


def _new_kv(rng, B, L):
    k = rng.standard_normal((B, L, 8, 128)).astype(np.float16)
    v = rng.standard_normal((B, L, 8, 128)).astype(np.float16)
    return k, v


def test_appended_token_reads_back_and_nothing_else_changes():
    m, pool, table, lens, free = _setup([16, 5, 33, 47])
    rng = np.random.default_rng(0)
    before = {(s, l): OA.gather_layer(pool, table[s], int(lens[s]), l)
              for s in range(4) for l in range(2)}
    k, v = _new_kv(rng, 4, 2)
    top, allocs, rejected = PG.append_step(pool, table, lens, free, free.size, k, v)
    assert rejected == []
    assert lens.tolist() == [17, 6, 34, 48]
    for s in range(4):
        for l in range(2):
            K, V = OA.gather_layer(pool, table[s], int(lens[s]), l)
            K0, V0 = before[(s, l)]
            assert np.array_equal(K[:, :-1], K0) and np.array_equal(V[:, :-1], V0)
            assert np.array_equal(K[:, -1], k[s, l].astype(np.float64))
            assert np.array_equal(V[:, -1], v[s, l].astype(np.float64))


def test_allocation_order_from_the_top_of_the_stack():
    m, pool, table, lens, free = _setup([16, 5, 32, 1])
    k, v = _new_kv(np.random.default_rng(1), 4, 2)
    top, allocs, rejected = PG.append_step(pool, table, lens, free, free.size, k, v)
    # sequences 0 (t=16) and 2 (t=32) open new blocks, in batch order
    assert [(s, b) for s, b, _ in allocs] == [(0, 1), (2, 2)]
    assert [p for _, _, p in allocs] == [int(free[-1]), int(free[-2])]
    assert top == free.size - 2
    assert table[0, 1] == free[-1] and table[2, 2] == free[-2]


def test_exhausted_stack_and_full_table_reject():
    m, pool, table, lens, free = _setup([16, 32, 48])
    k, v = _new_kv(np.random.default_rng(2), 3, 2)
    pool0 = pool.copy()
    top, allocs, rejected = PG.append_step(pool, table, lens, free, 1, k, v)
    assert [s for s, _, _ in allocs] == [0] and rejected == [1, 2] and top == 0
    assert lens.tolist() == [17, 32, 48]
    # only the allocated block changed
    diff = pool.view(np.uint16) != pool0.view(np.uint16)          # bitwise (spares hold NaN)
    changed = np.nonzero(diff.reshape(pool.shape[0], -1).any(axis=1))[0]
    assert changed.tolist() == [int(free[0])]
    # a full table row rejects even with free blocks
    m, pool, table, lens, free = _setup([16])
    table = table[:, :1]
    top, allocs, rejected = PG.append_step(pool, table, lens, free, free.size, *_new_kv(
        np.random.default_rng(3), 1, 2))
    assert rejected == [0] and lens.tolist() == [16]


def test_grow_keeps_history_and_adds_fresh_records():
    st = OS.init_state([2, 1], [7, 8])
    st, _ = OS.score_update(st, [np.array([1.0, 2.0]), np.array([3.0])], 0, OS.Policy(alpha=0.5))
    g = OS.grow(st, [3, 1])
    assert g.block.tolist() == [0, 1, 2, 0]
    assert g.seq_id.tolist() == [7, 7, 7, 8]
    np.testing.assert_array_equal(g.score[[0, 1, 3]], st.score)
    assert g.score[2] == 0.0 and g.t_touch[2] == OS.NEVER and g.tier[2] == OS.UNCLASSIFIED
    assert g.nblocks.tolist() == [3, 3, 3, 1]
    with pytest.raises(ValueError):
        OS.grow(st, [1, 1])


def test_append_rebuilds_a_cache_made_at_the_longer_length():
    """Take a cache made with lengths n+1, cut every sequence back to n (the last
    token's block returns to the free stack when it held only that token), and
    append the cut token: pool, table and decode are those of the original."""
    lens1 = [17, 32, 1, 48, 100]
    wl = W.custom("cut", 2, lens1, seed=21, spare_blocks=4)
    m = W.materialise(wl, "cpu")
    pool = m.pool.numpy().copy()
    table = m.table_host.astype(np.int64).copy()
    B, L = len(lens1), 2
    k = np.empty((B, L, 8, 128), np.float16)
    v = np.empty((B, L, 8, 128), np.float16)
    freed = []
    for s, n1 in enumerate(lens1):
        b, slot = divmod(n1 - 1, 16)
        pid = int(table[s, b])
        k[s] = pool[pid, :, 0, :, slot, :]
        v[s] = pool[pid, :, 1, :, slot, :]
        pool[pid, :, :, :, slot, :] = np.nan               # the cut slot forgets its token
        if slot == 0:
            freed.append(pid)
            table[s, b] = -1
    free = np.array(freed[::-1], dtype=np.int64)            # first needing sequence takes freed[0]
    lens = np.array([n - 1 for n in lens1], dtype=np.int64)
    top, allocs, rejected = PG.append_step(pool, table, lens, free, free.size, k, v)
    assert rejected == [] and top == 0
    assert lens.tolist() == lens1
    assert np.array_equal(table, m.table_host)
    live = np.unique(table[table >= 0])
    assert np.array_equal(pool[live].view(np.uint16), m.pool.numpy()[live].view(np.uint16))
    q = np.random.default_rng(5).standard_normal((B, L, 64, 128)).astype(np.float16)
    scale = 1.0 / np.sqrt(128.0)
    out_a, mass_a = OA.decode_step(q, pool, table, lens1, scale)
    out_b, mass_b = OA.decode_step(q, m.pool.numpy(), m.table_host, lens1, scale)
    assert np.array_equal(out_a, out_b)
    assert all(np.array_equal(x, y) for x, y in zip(mass_a, mass_b))


def test_sixteen_appends_fill_one_block_then_open_the_next():
    m, pool, table, lens, free = _setup([16, 3], spare=4)
    rng = np.random.default_rng(9)
    top = free.size
    opened = []
    for step in range(17):
        k, v = _new_kv(rng, 2, 2)
        top, allocs, rejected = PG.append_step(pool, table, lens, free, top, k, v)
        assert rejected == []
        opened += [(step, s, b) for s, b, _ in allocs]
    # sequence 0 opens block 1 at its first append and block 2 after 16 more;
    # sequence 1 (3 tokens) opens block 1 when it reaches 16 tokens (13th append)
    assert opened == [(0, 0, 1), (13, 1, 1), (16, 0, 2)]
    assert lens.tolist() == [33, 20]
    assert top == free.size - 3
