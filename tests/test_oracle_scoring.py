"""Pins for the oracle's normalise / EMA / touch / priority / tier."""
import json
import math
import os

import numpy as np
import pytest

from oracle import scoring as S

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _round_like(x, printed: str) -> str:
    decimals = len(printed.split(".")[1]) if "." in printed else 0
    return f"{x:.{decimals}f}"


def test_ema_worked_example():
    with open(os.path.join(GOLD, "ema_worked_example.json")) as f:
        g = json.load(f)
    for seq in g["sequences"]:
        e = g["initial_score"]
        for x, printed in zip(seq["attention"], seq["printed_score"]):
            e = float(S.ema(e, x, g["alpha"]))
            assert _round_like(e, printed) == printed, (seq["label"], x, e, printed)
    # the unrounded trajectory of the first token: 0.008, 0.0124, 0.01992
    e1 = S.ema(0.0, 0.04, 0.2)
    e2 = S.ema(e1, 0.03, 0.2)
    e3 = S.ema(e2, 0.05, 0.2)
    np.testing.assert_allclose([e1, e2, e3], [0.008, 0.0124, 0.01992], rtol=1e-12)


@pytest.mark.parametrize("alpha", [0.01, 0.05, 0.15, 0.2])
@pytest.mark.parametrize("c", [1.0, 0.37])
def test_ema_closed_form_on_constant_input(alpha, c):
    e = 0.0
    for t in range(40):
        e = float(S.ema(e, c, alpha))
        assert math.isclose(e, c * (1.0 - (1.0 - alpha) ** (t + 1)), rel_tol=1e-12)


def test_half_life_printed():
    with open(os.path.join(GOLD, "arithmetic.json")) as f:
        g = json.load(f)["half_life"]
    alpha = g["alpha"]
    e = [1.0]
    for _ in range(20):
        e.append(float(S.ema(e[-1], 0.0, alpha)))
    k = next(i for i, v in enumerate(e) if v < 0.5)
    assert k == 14 and e[13] > 0.5
    # log-linear crossing between the two steps that straddle one half
    cross = 13 + math.log(e[13] / 0.5) / math.log(e[13] / e[14])
    assert _round_like(cross, g["printed_steps"]) == g["printed_steps"]


def test_normalise_max_is_one_and_scale_free():
    rng = np.random.default_rng(1)
    mass = rng.uniform(0.1, 5.0, size=33)
    n = S.normalise(mass)
    assert n.max() == 1.0
    assert np.argmax(n) == np.argmax(mass)
    np.testing.assert_allclose(S.normalise(mass * 7.25), n, rtol=1e-15)
    assert np.all(S.normalise(np.zeros(4)) == 0.0)


def test_cut_point_inclusivity():
    pol = S.Policy(alpha=0.15)
    p = np.array([0.0, np.nextafter(0.3, 0), 0.3, np.nextafter(0.6, 0), 0.6, 1.0])
    assert S.tier_of(p, pol).tolist() == [2, 2, 1, 1, 0, 0]


def _closed_form_sets(nb, E, pol):
    """Tier sets for a sequence whose every block has score E, obtained by
    solving w_R (b + 1) / nb + w_E E + w_N [b < anchor] >= cut for b."""
    def first_block_at_least(cut, anchor_bonus):
        need = cut - pol.w_ema * E - anchor_bonus
        return max(0, math.ceil(nb * need / pol.w_recency) - 1)

    tiers = {}
    for b in range(nb):
        bonus = pol.w_anchor if b < pol.anchor_blocks else 0.0
        if b >= first_block_at_least(pol.t_high, bonus):
            tiers[b] = 0
        elif b >= first_block_at_least(pol.t_low, bonus):
            tiers[b] = 1
        else:
            tiers[b] = 2
    return tiers


@pytest.mark.parametrize("nb,alpha,steps,t0,t1", [
    # (blocks, alpha, steps, expected tier-0 count, tier-1 count)
    (64, 0.15, 10, 25, 39),
    (512, 0.15, 32, 405, 107),
    (8192, 0.05, 16, 0, 8192),
    (65536, 0.01, 4, 0, 0),
])
def test_constant_mass_tiers_closed_form(nb, alpha, steps, t0, t1):
    """With equal block mass every normalised input is 1, so after S steps
    E = 1 - (1 - alpha)^S and every label follows from the priority form."""
    pol = S.Policy(alpha=alpha)
    st = S.init_state([nb], [42], pol.anchor_blocks)
    for step in range(steps):
        st, stale = S.score_update(st, [np.full(nb, 3.0)], step, pol)
        assert not stale.any()
    E = 1.0 - (1.0 - alpha) ** steps
    np.testing.assert_allclose(st.score, E, rtol=1e-13)
    want = _closed_form_sets(nb, E, pol)
    p = st.priority
    away = (np.abs(p - pol.t_low) > 1e-9) & (np.abs(p - pol.t_high) > 1e-9)
    got = st.tier
    for b in range(nb):
        if away[b]:
            assert got[b] == want[b], (b, p[b])
    assert int((got == 0).sum()) == t0
    assert int((got == 1).sum()) == t1
    assert int((got == 2).sum()) == nb - t0 - t1


def test_small_table_of_labels():
    # 64 blocks, alpha 0.15, 10 steps: E = 0.803126; tier 0 = {0} U {40..63}
    pol = S.Policy(alpha=0.15)
    st = S.init_state([64], [0])
    for step in range(10):
        st, _ = S.score_update(st, [np.ones(64)], step, pol)
    assert abs(st.score[0] - 0.803126) < 5e-7
    t0 = set(np.nonzero(st.tier == 0)[0].tolist())
    assert t0 == {0} | set(range(40, 64))
    assert set(np.nonzero(st.tier == 1)[0].tolist()) == set(range(1, 40))


def test_priority_terms():
    pol = S.Policy(alpha=0.1)
    # last block has recency 1; block 0 of 4 has recency 1/4 plus the anchor
    p = S.priority(np.array([0.0, 0.0, 1.0]), np.array([0, 3, 3]), np.array([4, 4, 4]),
                   np.array([True, False, False]), pol)
    np.testing.assert_allclose(p, [0.25 * 0.25 + 0.20, 0.25, 0.25 + 0.55], rtol=1e-15)


def test_touch_count_and_timestamp():
    pol = S.Policy(alpha=0.15)
    st = S.init_state([3, 5], [10, 11])
    assert (st.t_touch == S.NEVER).all() and (st.touch_count == 0).all()
    assert (st.tier == S.UNCLASSIFIED).all()
    masses = [np.array([1.0, 2.0, 3.0]), np.arange(1.0, 6.0)]
    for step in range(7):
        st, stale = S.score_update(st, masses, step, pol)
        assert not stale.any()
    assert (st.touch_count == 7).all() and (st.t_touch == 6).all()
    # a step that does not advance leaves every record unchanged
    st2, stale = S.score_update(st, masses, 6, pol)
    assert stale.all()
    assert np.array_equal(st2.score, st.score)
    assert np.array_equal(st2.touch_count, st.touch_count)
    # identity keys
    assert st.seq_id.tolist() == [10, 10, 10, 11, 11, 11, 11, 11]
    assert st.block.tolist() == [0, 1, 2, 0, 1, 2, 3, 4]


def test_classify_without_update_is_pure():
    pol = S.Policy(alpha=0.15)
    st = S.init_state([6], [0])
    st, _ = S.score_update(st, [np.arange(1.0, 7.0)], 0, pol, do_classify=False)
    assert (st.tier == S.UNCLASSIFIED).all()
    c = S.classify(st, pol)
    np.testing.assert_allclose(
        c.priority, 0.25 * np.arange(1, 7) / 6 + 0.55 * 0.15 * np.arange(1, 7) / 6
        + 0.2 * (np.arange(6) == 0), rtol=1e-14)
    assert np.array_equal(c.score, st.score)


def test_decay_across_a_gap_closed_form():
    """A block touched at step 0 and next at step 5 decays by (1 - alpha)^5
    between the two touches (input 0 on the untouched steps)."""
    alpha, c5 = 0.15, 0.4
    st = S.init_state([1], [0])
    st, _ = S.score_update(st, [np.array([1.0])], 0, S.Policy(alpha=alpha))
    assert math.isclose(st.score[0], alpha * 1.0)
    # scores are normalised per sequence, so a one-block sequence always sees 1
    st5, _ = S.score_update(st, [np.array([c5])], 5, S.Policy(alpha=alpha))
    expect = alpha * 1.0 + (1 - alpha) ** 5 * (alpha * 1.0)
    assert math.isclose(st5.score[0], expect, rel_tol=1e-14)
    # decayed() between touches is the closed form
    for t in range(0, 6):
        assert math.isclose(float(S.decayed(st, t, alpha)[0]), alpha * (1 - alpha) ** t,
                            rel_tol=1e-14)


def test_printed_key_orders_like_the_decayed_score():
    """K = ln S_touch + t_touch * (-ln(1 - alpha)) orders records exactly as their
    decayed scores at any later step (RETRACTIONS Sec. 3)."""
    rng = np.random.default_rng(5)
    for alpha in (0.01, 0.05, 0.15, 0.5):
        st = S.init_state([200], [0])
        st.score = rng.uniform(1e-4, 1.0, 200)
        st.t_touch = rng.integers(0, 40, 200).astype(np.uint64)
        k = S.order_key(st, alpha)
        for t in (40, 41, 57, 100):
            d = S.decayed(st, t, alpha)
            # same order, and K - t * (-ln(1 - alpha)) is ln of the decayed score
            assert np.array_equal(np.argsort(k, kind="stable"), np.argsort(d, kind="stable"))
            np.testing.assert_allclose(k - t * (-math.log1p(-alpha)), np.log(d), rtol=0,
                                       atol=1e-10)


def test_stale_high_keys_mislead_a_lazy_heap():
    """The defect the printed key fixes: judged by stored scores, the block
    touched long ago looks hotter than it is; judged by the decayed score
    (or the key), it is the coldest."""
    alpha = 0.15
    st = S.init_state([2], [0])
    st.score = np.array([0.5, 0.3])
    st.t_touch = np.array([0, 30], dtype=np.uint64)
    assert np.argmin(st.score) == 1
    blocks, scores = S.eviction_candidates(st, 30, alpha)
    assert blocks[0] == 0
    assert math.isclose(scores[0], 0.5 * (1 - alpha) ** 30)
    assert np.argmin(S.order_key(st, alpha)) == 0


def test_eviction_candidates_ties_masks_and_pins():
    st = S.init_state([4, 3], [0, 1])
    st.score = np.array([0.2, 0.1, 0.1, 0.4, 0.3, 0.3, 0.9])
    st.t_touch = np.full(7, 10, dtype=np.uint64)
    st.tier = np.array([1, 0, 1, 1, 2, 2, 0], dtype=np.uint8)
    b, _ = S.eviction_candidates(st, 10, 0.1)
    assert b.tolist() == [1, 0]                       # ties go to the lowest block
    b, _ = S.eviction_candidates(st, 10, 0.1, exclude_pinned=True)
    assert b.tolist() == [2, 0]
    b, sc = S.eviction_candidates(st, 10, 0.1, active=[False, True])
    assert b.tolist() == [-1, 0] and sc[0] == np.inf
    st.tier[:] = 0
    b, _ = S.eviction_candidates(st, 10, 0.1, exclude_pinned=True)
    assert b.tolist() == [-1, -1]
    # a never-touched record (score 0) is the coldest
    st2 = S.init_state([3], [0])
    st2.score = np.array([0.3, 0.0, 0.2])
    st2.t_touch = np.array([5, S.NEVER, 5], dtype=np.uint64)
    assert S.eviction_candidates(st2, 6, 0.1)[0].tolist() == [1]


def test_empty_sequences_have_no_records_and_no_candidate():
    # R19: an empty sequence has no records; scoring and eviction skip it
    st = S.init_state([0, 3, 0, 2], [10, 11, 12, 13])
    assert st.score.size == 5
    st, stale = S.score_update(st, [np.zeros(0), np.array([1.0, 2.0, 4.0]), np.zeros(0),
                                    np.array([3.0, 3.0])], 0, S.Policy(alpha=0.5))
    assert not stale.any()
    np.testing.assert_allclose(st.score, [0.125, 0.25, 0.5, 0.5, 0.5])
    b, sc = S.eviction_candidates(st, 1, 0.5, nseq=4)
    assert b.tolist() == [-1, 0, -1, 0] and np.isinf(sc[[0, 2]]).all()
