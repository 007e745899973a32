"""Pins for the oracle's gather + decode attention + block mass.

Each test checks the oracle against something other than itself: a closed
form, a textbook special case, a pure-Python brute force, torch's fp64
scaled_dot_product_attention on an independently gathered K/V, or an
invariance the definition implies.
"""
import math

import numpy as np
import pytest
import torch

from oracle import attention as OA
import workload as W

SCALE = 1.0 / math.sqrt(128.0)


def _small(seq_lens, layers=1, seed=11, **kw):
    wl = W.custom("t", layers, seq_lens, seed=seed, **kw)
    m = W.materialise(wl, "cpu")
    q = W.make_query(m, 0)
    return m, q


def _loop_gather(pool, table_row, n, layer, kv_head):
    """Token-by-token gather, written independently of the oracle."""
    K = np.empty((n, 128))
    V = np.empty((n, 128))
    for t in range(n):
        pid = int(table_row[t // 16])
        K[t] = pool[pid, layer, 0, kv_head, t % 16].astype(np.float64)
        V[t] = pool[pid, layer, 1, kv_head, t % 16].astype(np.float64)
    return K, V


def test_q_zero_gives_uniform_weights_and_mean_of_values():
    m, q = _small([37, 80], layers=2)
    q = torch.zeros_like(q)
    pool = m.pool.numpy()
    out, masses = OA.decode_step(q.numpy(), pool, m.table_host, m.lens, SCALE)
    for s, n in enumerate(m.lens):
        for layer in range(2):
            for h in (0, 9, 63):
                _, V = _loop_gather(pool, m.table_host[s], n, layer, h // 8)
                np.testing.assert_allclose(out[s, layer, h], V.mean(axis=0), rtol=0, atol=1e-12)
        # every token carries 1/n of each (layer, head) softmax
        expect = np.array([min(16, n - 16 * b) for b in range(m.blocks[s])]) * 2 * 64 / n
        np.testing.assert_allclose(masses[s], expect, rtol=1e-12)


def test_one_hot_key_closed_form():
    n, hot, c = 50, 23, 8.0
    m, q = _small([n])
    pool = m.pool.clone()
    g = 3
    pid_hot = int(m.table_host[0, hot // 16])
    for b in range(m.blocks[0]):
        pool[int(m.table_host[0, b]), 0, 0, g] = 0.0
    pool[pid_hot, 0, 0, g, hot % 16] = 0.0
    pool[pid_hot, 0, 0, g, hot % 16, 5] = c
    q = torch.zeros_like(q)
    q[0, 0, 8 * g + 2, 5] = 1.0
    out, _ = OA.decode_step(q.numpy(), pool.numpy(), m.table_host, m.lens, SCALE)
    z = c * SCALE
    p_hot = math.exp(z) / (math.exp(z) + n - 1)
    _, V = _loop_gather(pool.numpy(), m.table_host[0], n, 0, g)
    others = (V.sum(axis=0) - V[hot]) / (n - 1)
    expect = p_hot * V[hot] + (1 - p_hot) * others
    np.testing.assert_allclose(out[0, 0, 8 * g + 2], expect, rtol=0, atol=1e-12)


def test_pure_python_brute_force():
    m, q = _small([21, 40], layers=2, seed=5)
    pool = m.pool.numpy()
    qn = q.numpy()
    out, masses = OA.decode_step(qn, pool, m.table_host, m.lens, SCALE)
    for s, n in enumerate(m.lens):
        mass = [0.0] * m.blocks[s]
        for layer in range(2):
            kv = [_loop_gather(pool, m.table_host[s], n, layer, g) for g in range(8)]
            for h in range(64):
                K, V = kv[h // 8]
                qh = [float(x) for x in qn[s, layer, h]]
                z = [SCALE * sum(qh[d] * K[t, d] for d in range(128)) for t in range(n)]
                mx = max(z)
                e = [math.exp(v - mx) for v in z]
                tot = sum(e)
                p = [v / tot for v in e]
                ref = [sum(p[t] * V[t, d] for t in range(n)) for d in range(128)]
                np.testing.assert_allclose(out[s, layer, h], ref, rtol=1e-12, atol=1e-12)
                for t in range(n):
                    mass[t // 16] += p[t]
        np.testing.assert_allclose(masses[s], mass, rtol=1e-12)


def test_against_torch_sdpa_fp64():
    m, q = _small([300, 129, 16], layers=3, seed=9)
    pool = m.pool.to(torch.float64)
    out, _ = OA.decode_step(q.numpy(), m.pool.numpy(), m.table_host, m.lens, SCALE)
    for s, n in enumerate(m.lens):
        tok = torch.arange(n)
        pids = torch.from_numpy(m.table_host[s].astype(np.int64))[tok // 16]
        for layer in range(3):
            K = pool[pids, layer, 0, :, tok % 16]          # [n][8][128]
            V = pool[pids, layer, 1, :, tok % 16]
            K = K.permute(1, 0, 2).repeat_interleave(8, dim=0).contiguous()  # [64][n][128]
            V = V.permute(1, 0, 2).repeat_interleave(8, dim=0).contiguous()
            qq = q[s, layer].to(torch.float64)[:, None, :]  # [64][1][128]
            ref = torch.nn.functional.scaled_dot_product_attention(
                qq[None], K[None], V[None], scale=SCALE)[0, :, 0]
            np.testing.assert_allclose(out[s, layer], ref.numpy(), rtol=1e-10, atol=1e-12)


def test_physical_permutation_is_bit_invariant():
    m, q = _small([100, 33], layers=2, seed=3, spare_blocks=6)
    pool = m.pool.numpy()
    P = pool.shape[0]
    perm = np.random.default_rng(0).permutation(P)
    pool2 = np.empty_like(pool)
    pool2[perm] = pool
    table2 = np.where(m.table_host >= 0, perm[np.maximum(m.table_host, 0)], -1)
    o1, m1 = OA.decode_step(q.numpy(), pool, m.table_host, m.lens, SCALE)
    o2, m2 = OA.decode_step(q.numpy(), pool2, table2, m.lens, SCALE)
    assert np.array_equal(o1, o2)
    for a, b in zip(m1, m2):
        assert np.array_equal(a, b)


def test_gqa_group_map():
    m, q = _small([64], layers=1, seed=4)
    pool = m.pool.numpy()
    o1, _ = OA.decode_step(q.numpy(), pool, m.table_host, m.lens, SCALE)
    g1, g2 = 2, 5
    pool_sw = pool.copy()
    pool_sw[:, :, :, [g1, g2]] = pool[:, :, :, [g2, g1]]
    o2, _ = OA.decode_step(q.numpy(), pool_sw, m.table_host, m.lens, SCALE)
    moved = set(range(8 * g1, 8 * g1 + 8)) | set(range(8 * g2, 8 * g2 + 8))
    for h in range(64):
        same = np.array_equal(o1[0, 0, h], o2[0, 0, h])
        assert same == (h not in moved), h
    # swapping the query groups as well restores the original outputs, swapped
    q_sw = q.clone()
    q_sw[0, 0, 8 * g1:8 * g1 + 8] = q[0, 0, 8 * g2:8 * g2 + 8]
    q_sw[0, 0, 8 * g2:8 * g2 + 8] = q[0, 0, 8 * g1:8 * g1 + 8]
    o3, _ = OA.decode_step(q_sw.numpy(), pool_sw, m.table_host, m.lens, SCALE)
    assert np.array_equal(o3[0, 0, 8 * g1:8 * g1 + 8], o1[0, 0, 8 * g2:8 * g2 + 8])
    assert np.array_equal(o3[0, 0, 8 * g2:8 * g2 + 8], o1[0, 0, 8 * g1:8 * g1 + 8])


@pytest.mark.parametrize("lens,layers", [([1024], 1), ([45, 16, 17], 2)])
def test_mass_sums_to_one_per_head_and_layer(lens, layers):
    m, q = _small(lens, layers=layers, seed=21)
    out, masses = OA.decode_step(q.numpy(), m.pool.numpy(), m.table_host, m.lens, SCALE)
    for s in range(len(lens)):
        assert masses[s].shape == (m.blocks[s],)
        assert np.all(masses[s] > 0)
        assert math.isclose(masses[s].sum(), 64 * layers, rel_tol=1e-12)
    # a single head's probabilities sum to one
    K, V = OA.gather_layer(m.pool.numpy(), m.table_host[0], lens[0], 0, kv_head=1)
    _, p = OA.attend_head(q.numpy()[0, 0, 9], K, V, SCALE)
    assert math.isclose(p.sum(), 1.0, rel_tol=1e-14)


def test_layer_range_splits_mass_additively():
    m, q = _small([70, 20], layers=3, seed=8)
    args = (q.numpy(), m.pool.numpy(), m.table_host, m.lens, SCALE)
    o_all, m_all = OA.decode_step(*args)
    o_a, m_a = OA.decode_step(*args, layer_begin=0, layer_end=1)
    o_b, m_b = OA.decode_step(*args, layer_begin=1, layer_end=3)
    for s in range(2):
        np.testing.assert_allclose(m_a[s] + m_b[s], m_all[s], rtol=1e-14)
    assert np.array_equal(o_a[:, 0], o_all[:, 0])
    assert np.isnan(o_a[:, 1:]).all()


def test_recipe_locality_shows_in_mass():
    """The anchor and recent-tail boost of the synthetic recipe must make
    block 0 and the last tenth hotter than the middle (sanity of inputs)."""
    m, q = _small([1024], layers=1, seed=0)
    _, masses = OA.decode_step(q.numpy(), m.pool.numpy(), m.table_host, m.lens, SCALE)
    mass = masses[0]
    middle = mass[8:50].mean()
    assert mass[0] > 1.1 * middle
    assert mass[-6:].mean() > 1.1 * middle


def test_saturated_logits_stay_finite():
    """A logit gap far beyond exp's range must give an exact one-hot weight
    (the softmax is evaluated relative to its largest logit)."""
    n, hot = 40, 17
    m, q = _small([n])
    pool = m.pool.clone()
    g = 6
    for b in range(m.blocks[0]):
        pool[int(m.table_host[0, b]), 0, 0, g] = 0.0
    pid_hot = int(m.table_host[0, hot // 16])
    pool[pid_hot, 0, 0, g, hot % 16, 0] = 60000.0
    q = torch.zeros_like(q)
    q[0, 0, 8 * g, 0] = 60000.0
    out, masses = OA.decode_step(q.numpy(), pool.numpy(), m.table_host, m.lens, SCALE)
    _, V = _loop_gather(pool.numpy(), m.table_host[0], n, 0, g)
    assert np.array_equal(out[0, 0, 8 * g], V[hot])
    assert np.isfinite(masses[0]).all()


def test_empty_sequence_gives_zero_rows_and_no_blocks():
    # R19: an empty sequence has no records and zero output rows, and the
    # other sequences of the batch are computed as if it were absent
    m = W.materialise(W.custom("empty", 2, [0, 40, 0, 17], seed=3, spare_blocks=4), "cpu")
    assert m.blocks == [0, 3, 0, 2] and m.total_blocks == 5
    q = np.random.default_rng(0).standard_normal((4, 2, 64, 128)).astype(np.float16)
    out, mass = OA.decode_step(q, m.pool.numpy(), m.table_host, m.lens, 0.088)
    assert np.all(out[[0, 2]] == 0) and mass[0].size == 0 and mass[2].size == 0
    out2, mass2 = OA.decode_step(q[[1, 3]], m.pool.numpy(), m.table_host[[1, 3]],
                                 [m.lens[1], m.lens[3]], 0.088)
    assert np.array_equal(out[[1, 3]], out2)
    assert all(np.array_equal(a, b) for a, b in zip([mass[1], mass[3]], mass2))


def test_threaded_runner_equals_decode_step_bit_for_bit():
    """oracle/runner.py only schedules attention.decode_layer / kivi.decode_layer
    over (sequence, layer) pieces: its outputs and masses are those of
    decode_step, bit for bit, for any thread count."""
    from oracle import kivi as KV
    from oracle import runner as OR
    rng = np.random.default_rng(11)
    B, L, nb_max = 3, 3, 12
    lens = [130, 16 * nb_max, 1]
    pool = rng.standard_normal((40, L, 2, 8, 16, 128)).astype(np.float16)
    table = np.stack([rng.permutation(40)[:nb_max] for _ in range(B)]).astype(np.int32)
    q = rng.standard_normal((B, L, 64, 128)).astype(np.float16)

    def host_layer(s, layer):
        nb = -(-lens[s] // 16)
        return pool[table[s, :nb], layer][:, None]

    for fmt, ref_fn in (("fp16", lambda: OA.decode_step(q, pool, table, lens, 0.1)),
                        ("kivi2", lambda: KV.decode_step(q, pool, table, lens, 0.1))):
        out_ref, mass_ref = ref_fn()
        for threads in (1, 3):
            out, mass, info = OR.decode_layers(q, host_layer, lens, range(L), 0.1, fmt,
                                               threads=threads, blas_threads=1)
            assert np.array_equal(out, out_ref)
            for a, b in zip(mass, mass_ref):
                assert np.array_equal(a, b)
            assert info["workers"] == threads
