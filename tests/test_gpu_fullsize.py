"""Full-size parity at the workloads' real sizes, in the launch configuration
bench.py times (library-chosen split, all layers in one call).

The fp64 oracle cannot run a whole 40-128 GiB step in a test, so each case
checks what it can compute one by one, plus properties that hold at any size:
  * sampled (sequence, layer, head) output rows against the oracle's row;
  * each sequence's block mass sums to layers x 64 (every softmax sums to 1);
  * the one-call block mass equals the sum of single-layer calls (GPU vs GPU);
  * the single-layer block mass of sampled layers against the oracle's;
  * the scoring step against the oracle's scoring fed the GPU's block mass
    (EMA, touch counts and timestamps, priorities and tiers).
"""
import math

import numpy as np
import pytest
import torch

import workload as W
from oracle import attention as OA
from oracle import kivi as KV
from oracle import scoring as OS
from paged_gqa_kv_amd import api
from paged_gqa_kv_amd.session import DecodeSession

from . import parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _host_layer(m, s, layer):
    """One layer of sequence s's blocks, in logical order, on the host."""
    nb = m.blocks[s]
    pids = m.block_table[s, :nb].long()
    return m.pool[pids, layer].cpu().numpy()[:, None]          # [nb][1][2][8][16][128]


def _run(name, alpha, steps=2, rows=8, oracle_layers=1, seqs_for_layer_mass=None,
         kv_format="fp16", pair=False):
    print(f"\n[case] full size {name} ({kv_format} KV{', paired' if pair else ''}), alpha {alpha}, "
          f"{steps} steps", flush=True)
    wl = W.WORKLOADS[name]
    if kv_format == "e4m3":
        wl = W.as_e4m3(wl)
    elif kv_format == "kivi2":
        wl = W.as_kivi2(wl)
    m = W.materialise(wl, DEV)
    torch.cuda.synchronize()
    L = m.num_layers
    sess = DecodeSession(m, pair_role="auto" if pair else None)
    pol = OS.Policy(alpha=alpha)
    gpol = api.policy(alpha)
    offsets = m.meta_offsets.cpu().numpy()
    state = OS.init_state(m.blocks, m.seq_ids.cpu().numpy())
    q = None
    for step in range(steps):
        q = W.make_query(m, step)
        sess.decode(q)
        mass = sess.mass.cpu().numpy().astype(np.float64)
        sess.score(step, gpol)
        masses = [mass[offsets[s]:offsets[s + 1]] for s in range(m.batch)]
        state, stale = OS.score_update(state, masses, step, pol)
        assert not stale.any()
    torch.cuda.synchronize()
    assert sess.status() == 0
    if pair:
        # the paired decode gives the unpaired decode's bits at the same split
        ref = DecodeSession(m, split_blocks=sess.split_blocks)
        ref.decode(q)
        torch.cuda.synchronize()
        assert torch.equal(ref.out.view(torch.int16), sess.out.view(torch.int16))
        assert torch.equal(ref.mass.view(torch.int32), sess.mass.view(torch.int32))
        assert ref.status() == 0
        del ref
        print(f"  paired decode bit-identical to the unpaired decode at split "
              f"{sess.split_blocks}", flush=True)
    err, near = P.check_records(sess.records(), state, pol)
    print(f"  scoring: max |dE| {err:.2e}, {near} labels inside the cut-point band", flush=True)

    # block mass of the last step sums to L x 64 per sequence
    for s in range(m.batch):
        tot = mass[offsets[s]:offsets[s + 1]].sum()
        assert math.isclose(tot, L * 64, rel_tol=2e-5), (s, tot)
        assert (mass[offsets[s]:offsets[s + 1]] > 0).all()

    # sampled output rows of the last step
    rng = np.random.default_rng(123)
    qh = q.cpu().numpy()
    out = sess.out.float().cpu().numpy().astype(np.float64)
    scale = 1.0 / math.sqrt(128.0)
    for _ in range(rows):
        s = int(rng.integers(m.batch))
        layer = int(rng.integers(L))
        h = int(rng.integers(64))
        host = _host_layer(m, s, layer)
        if kv_format == "kivi2":
            K16, V16 = KV._gather16(host, np.arange(m.blocks[s]), m.lens[s], 0)
            K, V = KV.kivi_kv(K16[h // 8], V16[h // 8], m.lens[s])
        else:
            K, V = OA.gather_layer(host, np.arange(m.blocks[s]), m.lens[s], 0, kv_head=h // 8,
                                   kv_format=kv_format)
        ref, _ = OA.attend_head(qh[s, layer, h], K, V, scale)
        e = np.abs(out[s, layer, h] - ref).max()
        lim = np.abs(ref).max()
        assert e <= P.OUT_RTOL * lim, (s, layer, h, e / lim)

    # one call vs the sum of single-layer calls, and oracle single-layer mass
    per = DecodeSession(m, layer_begin=0, layer_end=1)
    summed = torch.zeros_like(sess.mass)
    one_layer = {}
    sample_layers = set(int(x) for x in rng.choice(L, size=oracle_layers, replace=False))
    for layer in range(L):
        per.decode(q, layer_begin=layer, layer_end=layer + 1)
        summed += per.mass
        if layer in sample_layers:
            one_layer[layer] = per.mass.cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    assert per.status() == 0
    torch.testing.assert_close(summed, sess.mass, rtol=2e-5, atol=0)
    seqs = range(m.batch) if seqs_for_layer_mass is None else seqs_for_layer_mass
    for layer, gm in one_layer.items():
        for s in seqs:
            host = _host_layer(m, s, layer)
            if kv_format == "kivi2":
                _, ref = KV.decode_layer(qh[s, layer], host, np.arange(m.blocks[s]), m.lens[s],
                                         0, scale)
            else:
                _, ref = OA.decode_layer(qh[s, layer], host, np.arange(m.blocks[s]), m.lens[s],
                                         0, scale, kv_format)
            got = gm[offsets[s]:offsets[s + 1]]
            assert np.all(np.abs(got - ref) <= P.MASS_RTOL * ref + 1e-7 * ref.max()), (layer, s)
        print(f"  layer {layer}: single-layer block mass matches the oracle", flush=True)
    del sess, per, m
    torch.cuda.empty_cache()


def test_fullsize_128k_context():
    _run("decode-80L-128K", 0.05, steps=3, rows=12, oracle_layers=2)


def test_fullsize_128k_context_alpha_015():
    _run("decode-80L-128K", 0.15, steps=2, rows=4, oracle_layers=1)


def test_fullsize_shared_prefix_batch():
    _run("decode-80L-32xMixed-shared2K", 0.15, steps=2, rows=12, oracle_layers=1,
         seqs_for_layer_mass=[0, 7, 31])


def test_fullsize_shared_prefix_batch_paired():
    _run("decode-80L-32xMixed-shared2K", 0.15, steps=2, rows=8, oracle_layers=1,
         seqs_for_layer_mass=[0, 1, 30], pair=True)


def test_fullsize_shared_prefix_batch_e4m3_paired():
    _run("decode-80L-32xMixed-shared2K", 0.15, steps=2, rows=6, oracle_layers=1,
         seqs_for_layer_mass=[2, 3], kv_format="e4m3", pair=True)


def test_fullsize_1m_context():
    _run("decode-32L-1M", 0.01, steps=2, rows=6, oracle_layers=1)


def test_fullsize_128k_context_e4m3():
    _run("decode-80L-128K", 0.05, steps=2, rows=8, oracle_layers=1, kv_format="e4m3")


def test_fullsize_1m_context_e4m3():
    _run("decode-32L-1M", 0.15, steps=2, rows=4, oracle_layers=1, kv_format="e4m3")


def test_fullsize_128k_context_kivi2():
    _run("decode-80L-128K", 0.05, steps=2, rows=6, oracle_layers=1, kv_format="kivi2")


def test_fullsize_shared_prefix_batch_kivi2():
    _run("decode-80L-32xMixed-shared2K", 0.15, steps=2, rows=6, oracle_layers=1,
         seqs_for_layer_mass=[0, 13], kv_format="kivi2")
