"""GPU parity of lazy decay and eviction candidates.

The library orders records by the order-preserving key of the pages'
RETRACTIONS Sec. 3; the oracle takes a brute-force argmin of the decayed
score itself, so these tests are the audit that section describes.  Where
several blocks tie within rounding, the GPU's choice is checked to be one of
the minimal ones.
"""
import math

import numpy as np
import pytest
import torch

import workload as W
from oracle import scoring as OS
from paged_gqa_kv_amd import api
from paged_gqa_kv_amd.session import DecodeSession

from . import parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda"
REL = 1e-12


def _case(msg):
    print(f"\n[case] {msg}", flush=True)


def _state_from_records(rec, m):
    st = OS.init_state(m.blocks, m.seq_ids.cpu().numpy())
    st.score = rec["score"].astype(np.float64).copy()
    st.t_touch = rec["t_touch"].astype(np.uint64).copy()
    st.tier = rec["tier"].astype(np.uint8).copy()
    return st


def _audit(m, rec, now, alpha, active, exclude_pinned, blk, key):
    st = _state_from_records(rec, m)
    ref_blk, ref_score = OS.eviction_candidates(st, now, alpha, active, exclude_pinned)
    d = OS.decayed(st, now, alpha)
    offs = m.meta_offsets.cpu().numpy()
    c = -math.log1p(-alpha)
    for s in range(m.batch):
        g = int(blk[s])
        if ref_blk[s] < 0:
            assert g == -1 and math.isinf(key[s]) and key[s] > 0, s
            continue
        assert g >= 0, s
        rows = np.arange(offs[s], offs[s + 1])
        got_score = d[offs[s] + g]
        # valid: the GPU's block is minimal within rounding, and eligible
        assert got_score <= ref_score[s] * (1 + REL) + 1e-300, (s, g, got_score, ref_score[s])
        if exclude_pinned:
            assert st.tier[offs[s] + g] != 0
        # unique: equal to the oracle's choice unless another block ties
        others = d[rows] <= ref_score[s] * (1 + REL)
        if others.sum() == 1:
            assert g == ref_blk[s], (s, g, ref_blk[s])
        # the returned key is ln of the decayed score plus now * (-ln(1 - alpha))
        if got_score > 0:
            assert math.isclose(key[s] - now * c, math.log(got_score), rel_tol=0, abs_tol=1e-9)
        else:
            assert key[s] == -math.inf


def test_gap_aware_score_update():
    _case("steps 0, 1, 2 then 7: records decay over the untouched steps")
    wl = W.custom("gap", 2, [300, 900, 40], seed=21)
    m = W.materialise(wl, DEV)
    h = P.host(m)
    pol = OS.Policy(alpha=0.15)
    gpol = api.policy(0.15)
    sess = DecodeSession(m)
    state = OS.init_state(m.blocks, m.seq_ids.cpu().numpy())
    for step in (0, 1, 2, 7, 8):
        q = W.make_query(m, step)
        sess.step(q, step, gpol)
        _, mass_ref = P.oracle_decode(h, q)
        state, _ = OS.score_update(state, mass_ref, step, pol)
        P.check_records(sess.records(), state, pol)
    assert sess.status() == 0


@pytest.mark.parametrize("exclude_pinned", [0, 1])
def test_eviction_candidates_after_decode(exclude_pinned):
    _case(f"candidates after 4 decode steps, exclude_pinned={exclude_pinned}")
    wl = W.custom("evict", 2, [1024, 333, 2049, 16], seed=5)
    m = W.materialise(wl, DEV)
    sess = DecodeSession(m)
    alpha = 0.15
    for step in range(4):
        sess.step(W.make_query(m, step), step, api.policy(alpha))
    for now, active in ((3, None), (9, [1, 0, 1, 1])):
        act = None if active is None else torch.tensor(active, dtype=torch.uint8, device=DEV)
        blk, key = sess.evict_candidates(now, alpha, act, exclude_pinned)
        torch.cuda.synchronize()
        _audit(m, sess.records(), now, alpha, active, bool(exclude_pinned),
               blk.cpu().numpy(), key.cpu().numpy())
    assert sess.status() == 0


@pytest.mark.parametrize("alpha", [0.01, 0.05, 0.15, 0.5])
def test_eviction_audit_on_random_states(alpha):
    _case(f"brute-force audit on random record states, alpha={alpha}")
    wl = W.custom("audit", 1, [16 * 3000, 16 * 257, 16 * 1, 16 * 700, 16 * 64], seed=9)
    m = W.materialise(wl, DEV)
    sess = DecodeSession(m)
    rng = np.random.default_rng(int(alpha * 1000))
    for trial in range(3):
        rec = sess.records().copy()
        n = rec.size
        rec["score"] = rng.uniform(1e-6, 1.0, n)
        rec["t_touch"] = rng.integers(0, 50, n).astype(np.uint64)
        rec["tier"] = rng.integers(0, 3, n).astype(np.uint8)
        never = rng.random(n) < 0.001 * trial
        rec["t_touch"][never] = OS.NEVER
        rec["score"][never] = 0.0
        # a few exact ties
        rec["score"][:5] = 0.25
        rec["t_touch"][:5] = 3
        sess.meta[:n].copy_(torch.from_numpy(rec.view(np.uint8).reshape(n, 64)).to(DEV))
        active = (rng.random(m.batch) < 0.8).astype(np.uint8)
        act = torch.from_numpy(active).to(DEV)
        for exclude in (0, 1):
            blk, key = sess.evict_candidates(60, alpha, act, exclude)
            torch.cuda.synchronize()
            _audit(m, rec, 60, alpha, active.astype(bool), bool(exclude), blk.cpu().numpy(),
                   key.cpu().numpy())
    assert sess.status() == 0


def test_future_touch_is_skipped_and_reported():
    _case("records touched after `now` are skipped")
    wl = W.custom("future", 1, [64, 64], seed=2)
    m = W.materialise(wl, DEV)
    sess = DecodeSession(m)
    rec = sess.records().copy()
    rec["score"] = np.linspace(0.9, 0.1, rec.size)
    rec["t_touch"] = 5
    rec["t_touch"][3] = 100          # touched after `now`: must be skipped
    rec["score"][3] = 1e-9           # ... although it is the coldest of its sequence
    rec["tier"] = 1
    sess.meta[:rec.size].copy_(torch.from_numpy(rec.view(np.uint8).reshape(rec.size, 64)).to(DEV))
    blk, key = sess.evict_candidates(10, 0.1)
    torch.cuda.synchronize()
    _audit(m, rec, 10, 0.1, None, False, blk.cpu().numpy(), key.cpu().numpy())
    assert int(blk[0]) == 2           # blocks 0..3; block 3 (coldest) is skipped
    assert sess.status() & api._abi.KVS_DEV_STALE_STEP
