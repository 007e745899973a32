"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Sizes here run the oracle in seconds yet span several splits, ragged last
blocks and length-1 sequences.  Every test prints the case it runs first.
"""
import numpy as np
import pytest
import torch

import workload as W
from oracle import attention as OA
from oracle import scoring as OS
from paged_gqa_kv_amd import api
from paged_gqa_kv_amd.session import DecodeSession

from . import parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _case(msg):
    print(f"\n[case] {msg}", flush=True)


def _run_pipeline(m, alpha, steps, split_blocks=0, check_decode_steps=None, seqs=None,
                  score_seqs=None):
    """Run `steps` decode + score steps on the GPU and the oracle side by side."""
    sess = DecodeSession(m, split_blocks=split_blocks)
    h = P.host(m)
    pol = OS.Policy(alpha=alpha)
    gpol = api.policy(alpha)
    offsets = m.meta_offsets.cpu().numpy()
    state = OS.init_state(m.blocks, m.seq_ids.cpu().numpy(), pol.anchor_blocks)
    score_seqs = list(range(m.batch)) if score_seqs is None else score_seqs
    rows = np.concatenate([np.arange(offsets[s], offsets[s + 1]) for s in score_seqs])
    worst = dict(out=0.0, mass=0.0)
    for step in range(steps):
        q = W.make_query(m, step)
        sess.step(q, step, gpol)
        torch.cuda.synchronize()
        need_decode = check_decode_steps is None or step in check_decode_steps
        sub = sorted(set(score_seqs) | (set(range(m.batch)) if need_decode else set()))
        # oracle decode of the sequences this step needs
        qh = q.cpu().numpy()
        h_sub = dict(h, table=h["table"][sub], lens=[h["lens"][s] for s in sub])
        out_ref, mass_ref = P.oracle_decode(h_sub, qh[sub])
        if need_decode:
            worst["out"] = max(worst["out"], P.check_out(sess.out[sub], out_ref,
                                                        range(m.num_layers)))
            worst["mass"] = max(worst["mass"], P.check_mass(sess.mass, mass_ref,
                                                           offsets[sub]))
        masses = [None] * m.batch
        for k, s in enumerate(sub):
            masses[s] = mass_ref[k]
        for s in range(m.batch):
            if masses[s] is None:  # not scored against the oracle: any positive vector
                masses[s] = np.ones(m.blocks[s])
        state, stale = OS.score_update(state, masses, step, pol)
        assert not stale.any()
        P.check_records(sess.records(), state, pol, rows=rows)
    assert sess.status() == 0
    return sess, worst


def test_tiny_workload_all_steps():
    _case("decode-1L-1K, 10 steps, alpha 0.15")
    m = W.materialise(W.WORKLOADS["decode-1L-1K"], DEV)
    _, worst = _run_pipeline(m, 0.15, 10)
    print(worst)


@pytest.mark.parametrize("split_blocks", [4, 16, 64])
def test_ragged_batch(split_blocks):
    _case(f"ragged lengths, 2 layers, split_blocks={split_blocks}")
    wl = W.custom("ragged", 2, [1, 15, 16, 17, 37, 300, 1000, 2049], seed=31, spare_blocks=9)
    m = W.materialise(wl, DEV)
    _run_pipeline(m, 0.05, 3, split_blocks=split_blocks)


def test_shared_prefix_and_odd_lengths():
    _case("shared 96-token prefix, 3 layers, mixed lengths")
    wl = W.custom("shared", 3, [40, 96, 500, 129, 1200], seed=12, shared_prefix_tokens=96)
    m = W.materialise(wl, DEV)
    assert m.refcount.max() > 1
    _run_pipeline(m, 0.15, 4, split_blocks=8)


def test_4L_8x8K_workload():
    _case("decode-4L-8x8K, 32 steps; decode parity at steps 0 and 31 on all sequences; "
          "scores of sequences 0 and 5 over all steps")
    m = W.materialise(W.WORKLOADS["decode-4L-8x8K"], DEV)
    _, worst = _run_pipeline(m, 0.15, 32, check_decode_steps={0, 31}, score_seqs=[0, 5])
    print(worst)


def _bits(t):
    return t.detach().contiguous().view(torch.uint8).cpu()


def test_physical_permutation_gives_identical_bits():
    _case("permutation invariance, 2 layers, 3 sequences")
    wl = W.custom("perm", 2, [700, 64, 333], seed=5, spare_blocks=20)
    m = W.materialise(wl, DEV)
    q = W.make_query(m, 0)
    s1 = DecodeSession(m, split_blocks=16)
    s1.decode(q)
    P_ = m.pool_blocks
    perm = torch.randperm(P_, generator=torch.Generator().manual_seed(1)).to(DEV)
    pool2 = torch.empty_like(m.pool)
    pool2[perm] = m.pool
    table2 = torch.where(m.block_table >= 0, perm[m.block_table.clamp(min=0).long()].int(),
                         m.block_table)
    m2 = type(m)(**{**m.__dict__, "pool": pool2, "block_table": table2})
    s2 = DecodeSession(m2, split_blocks=16)
    s2.decode(q)
    torch.cuda.synchronize()
    assert torch.equal(_bits(s1.out), _bits(s2.out))
    assert torch.equal(_bits(s1.mass), _bits(s2.mass))


def test_run_to_run_determinism():
    _case("determinism, decode-1L-1K and a 3-layer ragged batch")
    for wl in (W.WORKLOADS["decode-1L-1K"], W.custom("det", 3, [513, 47, 2000], seed=2)):
        m = W.materialise(wl, DEV)
        outs = []
        for _ in range(2):
            s = DecodeSession(m)
            for step in range(3):
                s.step(W.make_query(m, step), step, api.policy(0.15))
            torch.cuda.synchronize()
            outs.append((_bits(s.out), _bits(s.mass), _bits(s.meta)))
        for a, b in zip(*outs):
            assert torch.equal(a, b)


def test_record_save_restore_is_bit_exact():
    _case("records saved after step 2 and restored into a fresh session")
    wl = W.custom("resume", 2, [400, 90], seed=8)
    m = W.materialise(wl, DEV)
    pol = api.policy(0.05)
    full = DecodeSession(m)
    saved = None
    for step in range(6):
        full.step(W.make_query(m, step), step, pol)
        if step == 2:
            saved = full.meta.clone()
    resumed = DecodeSession(m)
    resumed.meta.copy_(saved)
    for step in range(3, 6):
        resumed.step(W.make_query(m, step), step, pol)
    torch.cuda.synchronize()
    assert torch.equal(_bits(full.meta), _bits(resumed.meta))


def test_layer_ranges_accumulate():
    _case("per-layer calls with accumulate vs one call, 3 layers")
    wl = W.custom("acc", 3, [300, 1000], seed=4)
    m = W.materialise(wl, DEV)
    q = W.make_query(m, 0)
    one = DecodeSession(m, split_blocks=16)
    one.decode(q)
    per = DecodeSession(m, split_blocks=16)
    for layer in range(3):
        per.decode(q, accumulate=int(layer > 0), layer_begin=layer, layer_end=layer + 1)
    torch.cuda.synchronize()
    assert torch.equal(_bits(one.out), _bits(per.out))
    torch.testing.assert_close(per.mass, one.mass, rtol=1e-6, atol=0)
    assert one.status() == 0 and per.status() == 0


def test_classify_entry_point_and_tiers_out():
    _case("score_update(classify=0) then classify with tiers_out")
    wl = W.custom("cls", 2, [333, 64, 1600], seed=9)
    m = W.materialise(wl, DEV)
    pol = OS.Policy(alpha=0.15)
    gpol = api.policy(0.15)
    sess = DecodeSession(m)
    h = P.host(m)
    state = OS.init_state(m.blocks, m.seq_ids.cpu().numpy())
    for step in range(4):
        q = W.make_query(m, step)
        sess.decode(q)
        sess.score(step, gpol, classify=0)
        _, mass_ref = P.oracle_decode(h, q)
        state, _ = OS.score_update(state, mass_ref, step, pol, do_classify=False)
    rec = sess.records()
    assert (rec["tier"] == 0xFF).all()
    tiers = torch.full((m.total_blocks,), 7, dtype=torch.uint8, device=DEV)
    sess.classify(gpol, tiers)
    torch.cuda.synchronize()
    ref = OS.classify(state, pol)
    P.check_records(sess.records(), ref, pol)
    assert np.array_equal(tiers.cpu().numpy(), sess.records()["tier"])


def test_scoring_is_exact_given_the_same_mass():
    _case("K3 alone: oracle scoring fed the GPU's block mass")
    wl = W.custom("k3", 2, [2000, 50, 777], seed=13)
    m = W.materialise(wl, DEV)
    pol = OS.Policy(alpha=0.05)
    gpol = api.policy(0.05)
    sess = DecodeSession(m)
    offsets = m.meta_offsets.cpu().numpy()
    state = OS.init_state(m.blocks, m.seq_ids.cpu().numpy())
    for step in range(5):
        sess.decode(W.make_query(m, step))
        mass = sess.mass.cpu().numpy().astype(np.float64)
        sess.score(step, gpol)
        masses = [mass[offsets[s]:offsets[s + 1]] for s in range(m.batch)]
        state, _ = OS.score_update(state, masses, step, pol)
    rec = sess.records()
    assert np.abs(rec["score"] - state.score).max() <= 1e-13
    assert np.abs(rec["priority"] - state.priority).max() <= 1e-13
    near = np.minimum(np.abs(state.priority - 0.3), np.abs(state.priority - 0.6)) < 1e-12
    assert np.array_equal(rec["tier"][~near], state.tier[~near])
    assert np.array_equal(rec["touch_count"], state.touch_count)
    assert np.array_equal(rec["t_touch"], state.t_touch)


def test_device_status_bits():
    _case("bad block id, over-long sequence and a stale step set status bits")
    wl = W.custom("bad", 1, [64, 64], seed=3, spare_blocks=2)
    m = W.materialise(wl, DEV)
    q = W.make_query(m, 0)
    bad_table = m.block_table.clone()
    bad_table[1, 2] = m.pool_blocks + 5          # out of the pool: skipped
    m_bad = type(m)(**{**m.__dict__, "block_table": bad_table})
    s = DecodeSession(m_bad)
    s.decode(q)
    assert s.status() & api._abi.KVS_DEV_BAD_BLOCK_ID
    # sequence 0 is untouched by the bad entry of sequence 1
    h = P.host(m)
    out_ref, mass_ref = P.oracle_decode(dict(h, table=h["table"][:1], lens=h["lens"][:1]),
                                        q[:1])
    P.check_out(s.out[:1], out_ref, [0])
    assert torch.isfinite(s.out).all()

    long_lens = m.seq_lens.clone()
    long_lens[0] = 16 * m.max_blocks + 1
    m_long = type(m)(**{**m.__dict__, "seq_lens": long_lens})
    s2 = DecodeSession(m_long)
    s2.decode(q)
    assert s2.status() & api._abi.KVS_DEV_BAD_SEQ_LEN

    s3 = DecodeSession(m)
    s3.step(q, 4, api.policy(0.15))
    before = s3.meta.clone()
    s3.score(4, api.policy(0.15))               # same step again: stale
    torch.cuda.synchronize()
    assert s3.status() & api._abi.KVS_DEV_STALE_STEP
    assert torch.equal(_bits(before), _bits(s3.meta))


def test_unused_pool_blocks_are_nan_and_never_read():
    _case("NaN-poisoned spare blocks stay out of the result")
    m = W.materialise(W.WORKLOADS["decode-1L-1K"], DEV)
    assert torch.isnan(m.pool).any()
    s = DecodeSession(m)
    s.step(W.make_query(m, 0), 0, api.policy(0.15))
    torch.cuda.synchronize()
    assert torch.isfinite(s.out).all() and torch.isfinite(s.mass).all()
    assert np.isfinite(s.records()["score"]).all()


def test_empty_sequences_in_the_batch():
    """R19: empty sequences have no records and zero output rows; the rest of the
    batch is unaffected; an append gives an empty sequence its first block."""
    _case("batch with empty sequences: decode, score, evict, then append one token")
    from oracle import paging as PG
    wl = W.custom("empty", 2, [0, 40, 0, 17, 300], seed=6, spare_blocks=10)
    m = W.materialise(wl, DEV, extra_blocks=2)
    assert m.blocks[0] == 0 and m.blocks[2] == 0
    sess = DecodeSession(m)
    h = P.host(m)
    pol = OS.Policy(alpha=0.15)
    gpol = api.policy(0.15)
    offsets = m.meta_offsets.cpu().numpy()
    state = OS.init_state(m.blocks, m.seq_ids.cpu().numpy())
    live_rows = np.concatenate([offsets[s] + np.arange(nb) for s, nb in enumerate(m.blocks)])
    for step in range(2):
        q = W.make_query(m, step)
        sess.step(q, step, gpol)
        torch.cuda.synchronize()
        out_ref, mass_ref = P.oracle_decode(h, q)
        assert torch.count_nonzero(sess.out[[0, 2]]) == 0
        P.check_out(sess.out, out_ref, range(2), seqs=[1, 3, 4])
        P.check_mass(sess.mass, mass_ref, offsets, seqs=[1, 3, 4])
        state, _ = OS.score_update(state, mass_ref, step, pol)
        P.check_records(sess.records()[live_rows], state, pol)
    blk, _ = sess.evict_candidates(1, 0.15)
    ref_blk, _ = OS.eviction_candidates(state, 1, 0.15, nseq=m.batch)
    assert blk.cpu().tolist() == ref_blk.tolist() and ref_blk[0] == -1 and ref_blk[2] == -1
    # one append: the empty sequences open block 0
    pool_h = m.pool.cpu().numpy().copy()
    table_h = m.table_host.astype(np.int64).copy()
    lens_h = np.array(m.lens, dtype=np.int64)
    free_h = m.free_stack.astype(np.int64).copy()
    k, v = W.new_token_kv(m, 9)
    sess.append(k, v)
    top, allocs, rejected = PG.append_step(pool_h, table_h, lens_h, free_h, int(free_h.size),
                                           k.cpu().numpy(), v.cpu().numpy())
    assert rejected == [] and [s for s, b, _ in allocs][:2] == [0, 2]
    q = W.make_query(m, 9)
    sess.decode(q)
    torch.cuda.synchronize()
    assert m.seq_lens.cpu().tolist() == lens_h.tolist()
    out_ref, mass_ref = P.oracle_decode(dict(pool=pool_h, table=table_h, lens=list(lens_h)), q)
    P.check_out(sess.out, out_ref, range(2))
    P.check_mass(sess.mass, mass_ref, offsets)
    assert sess.status() == 0


def test_uniform_attention_and_alpha_one_closed_forms():
    """q = 0: every logit is 0, so each head attends uniformly (out = mean of V)
    and a block's mass is proportional to its token count; with alpha = 1 the
    EMA equals the normalised mass: token count / the sequence's largest block
    token count (1 for full blocks; a lone partial block is its own maximum)."""
    _case("q = 0 and alpha = 1: closed-form outputs, masses and scores")
    wl = W.custom("uniform", 2, [40, 100, 16, 5], seed=14)
    m = W.materialise(wl, DEV)
    q = torch.zeros((m.batch, 2, 64, 128), dtype=torch.float16, device=DEV)
    sess = DecodeSession(m, split_blocks=4)
    sess.step(q, 0, api.policy(1.0))
    torch.cuda.synchronize()
    h = P.host(m)
    offsets = m.meta_offsets.cpu().numpy()
    out = sess.out.float().cpu().numpy()
    mass = sess.mass.cpu().numpy().astype(np.float64)
    rec = sess.records()
    for s, n in enumerate(m.lens):
        for layer in range(2):
            K, V = OA.gather_layer(h["pool"], h["table"][s], n, layer)
            mean = V.mean(axis=1)                                   # [8][128]
            ref = np.repeat(mean, 8, axis=0)                        # head h reads KV head h // 8
            assert np.abs(out[s, layer] - ref).max() <= 2e-3 * np.abs(ref).max()
        nb = -(-n // 16)
        counts = np.array([min(16, n - 16 * b) for b in range(nb)], dtype=np.float64)
        got = mass[offsets[s]:offsets[s] + nb]
        np.testing.assert_allclose(got, 2 * 64 * counts / n, rtol=1e-6)
        E = rec["score"][offsets[s]:offsets[s] + nb]
        np.testing.assert_allclose(E, counts / counts.max(), rtol=0, atol=1e-6)
        assert np.all(E[counts == counts.max()] == 1.0)
    assert sess.status() == 0


def test_large_batch_of_short_sequences():
    """3,000 sequences of 0..80 tokens in one call: per-sequence grids far past
    one work-group, decode of a sample against the oracle, scoring of every
    record against the oracle fed the GPU's mass, and eviction candidates."""
    _case("batch of 3,000 short sequences, 1 layer, 2 steps")
    rng = np.random.default_rng(77)
    lens = [int(x) for x in rng.integers(0, 81, size=3000)]
    m = W.materialise(W.custom("many", 1, lens, seed=14, spare_blocks=16), DEV)
    sess = DecodeSession(m)
    h = P.host(m)
    pol = OS.Policy(alpha=0.15)
    gpol = api.policy(0.15)
    offsets = m.meta_offsets.cpu().numpy()
    state = OS.init_state(m.blocks, m.seq_ids.cpu().numpy())
    sample = sorted(set(int(x) for x in rng.choice(3000, size=60, replace=False)) | {0, 2999})
    sample = [s for s in sample if lens[s] > 0]
    live_rows = np.concatenate([offsets[s] + np.arange(nb) for s, nb in enumerate(m.blocks)])
    for step in range(2):
        q = W.make_query(m, step)
        sess.step(q, step, gpol)
        torch.cuda.synchronize()
        h_sub = dict(h, table=h["table"][sample], lens=[lens[s] for s in sample])
        out_ref, mass_ref = P.oracle_decode(h_sub, q.cpu().numpy()[sample])
        P.check_out(sess.out[sample], out_ref, range(1))
        P.check_mass(sess.mass, mass_ref, offsets[sample])
        gpu_mass = sess.mass.cpu().numpy().astype(np.float64)
        masses = [gpu_mass[offsets[s]:offsets[s] + m.blocks[s]] for s in range(m.batch)]
        state, stale = OS.score_update(state, masses, step, pol)
        assert not stale.any()
        P.check_records(sess.records()[live_rows], state, pol)
    blk, _ = sess.evict_candidates(1, 0.15)
    ref_blk, _ = OS.eviction_candidates(state, 1, 0.15, nseq=m.batch)
    assert blk.cpu().tolist() == ref_blk.tolist()
    assert sess.status() == 0


@pytest.mark.parametrize("fmt,split_blocks,paired", [("fp16", 1024, False), ("e4m3", 1024, False),
                                                     ("fp16", 512, True), ("e4m3", 512, True)])
def test_longest_splits_with_a_one_block_tail(fmt, split_blocks, paired):
    """The largest split sizes the entry points take, over sequences whose last
    split holds one block (and a partial one), against the oracle."""
    _case(f"{fmt}, split {split_blocks}, paired {paired}: 2,049- and 1,025-block sequences")
    lens = [16 * 2048 + 5, 16 * 1024 + 16, 300, 16 * 1024 + 1]
    wl = W.custom("long", 1, lens, seed=23, spare_blocks=8, shared_prefix_tokens=4096)
    if fmt == "e4m3":
        wl = W.as_e4m3(wl)
    m = W.materialise(wl, DEV)
    sess = DecodeSession(m, split_blocks=split_blocks, pair_role="auto" if paired else None)
    q = W.make_query(m, 3)
    sess.decode(q)
    torch.cuda.synchronize()
    assert sess.status() == 0
    out_ref, mass_ref = P.oracle_decode(P.host(m), q)
    P.check_out(sess.out, out_ref, range(1))
    P.check_mass(sess.mass, mass_ref, m.meta_offsets.cpu().numpy())
