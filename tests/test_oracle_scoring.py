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
