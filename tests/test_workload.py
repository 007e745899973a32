"""Host-side checks of the seeded synthetic workloads."""
import numpy as np
import torch

import workload as W


def test_tables_are_injective_and_spare_blocks_are_nan():
    wl = W.WORKLOADS["decode-1L-1K"]
    m = W.materialise(wl, "cpu")
    assert m.pool.shape == (256, 1, 2, 8, 16, 128)
    assert m.pool.dtype == torch.float16
    row = m.table_host[0]
    assert row.shape == (64,)
    assert len(set(row.tolist())) == 64 and row.min() >= 0 and row.max() < 256
    used = np.zeros(256, bool)
    used[row] = True
    assert torch.isnan(m.pool[torch.from_numpy(np.nonzero(~used)[0])]).all()
    assert not torch.isnan(m.pool[torch.from_numpy(row.astype(np.int64))]).any()
    assert m.meta_offsets.tolist() == [0, 64]
    assert m.total_blocks == 64


def test_structure_is_device_independent_and_seeded():
    wl = W.custom("a", 2, [40, 17, 100], seed=3)
    m1 = W.materialise(wl, "cpu")
    m2 = W.materialise(wl, "cpu")
    assert np.array_equal(m1.table_host, m2.table_host)
    assert torch.equal(m1.pool.view(torch.int16), m2.pool.view(torch.int16))
    assert torch.equal(W.make_query(m1, 2), W.make_query(m2, 2))
    assert not torch.equal(W.make_query(m1, 2), W.make_query(m1, 3))
    assert m1.blocks == [3, 2, 7]
    assert (m1.table_host[1, 2:] == -1).all()


def test_shared_prefix_refcounts():
    wl = W.custom("sh", 1, [40, 64, 20], shared_prefix_tokens=32, seed=5)
    m = W.materialise(wl, "cpu")
    t = m.table_host
    # the first two blocks of the two longer sequences and the first two
    # blocks of the 20-token sequence are the same physical blocks
    assert t[0, 0] == t[1, 0] == t[2, 0]
    assert t[0, 1] == t[1, 1] == t[2, 1]
    assert m.refcount[t[0, 0]] == 3 and m.refcount[t[0, 1]] == 3
    private = [t[0, 2], t[1, 2], t[1, 3]]
    assert len(set(private)) == 3 and all(m.refcount[p] == 1 for p in private)
    assert m.unique_blocks == 2 + 1 + 2


def test_query_boost_direction():
    wl = W.custom("b", 2, [32], seed=1, q_boost=4.0)
    m = W.materialise(wl, "cpu")
    q = W.make_query(m, 0).float()
    # the projection of each query on its group's u is centred near +4
    proj = torch.einsum("lgkd,lgd->lgk", q[0].reshape(2, 8, 8, 128), m.u)
    assert abs(proj.mean().item() - 4.0) < 0.5


def test_mixed_lengths_rounded_to_blocks():
    wl = W.WORKLOADS["decode-80L-32xMixed-shared2K"]
    lens = wl.lengths()
    assert len(lens) == 32
    assert all(n % 16 == 0 and 1024 <= n <= 32768 for n in lens)
    assert lens == wl.lengths()
