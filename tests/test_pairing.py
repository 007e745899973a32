"""Host logic of the paired decode: pair_plan's links and the count of tokens
the paired kernel loads (pair_loaded_tokens), against closed forms."""
import numpy as np
import pytest

import workload as W
from workload.recipe import _layout
from paged_gqa_kv_amd.session import pair_loaded_tokens, pair_plan


def _tables(lens, shared_tokens, seed=3):
    wl = W.custom("pairs", 1, lens, seed=seed, spare_blocks=2, shared_prefix_tokens=shared_tokens)
    lens, blocks, _, _, table, _, _, _ = _layout(wl)
    return list(lens), blocks, table


def test_pair_plan_links_sharers_in_batch_order():
    lens = [700, 100, 0, 333, 288, 1000, 40]
    _, blocks, table = _tables(lens, 288)
    role = pair_plan(table, blocks)
    # sharers (non-empty) in batch order: 0 1 3 4 5 6 -> pairs (0,1) (3,4) (5,6)
    assert role.tolist() == [1, -2, -1, 4, -5, 6, -7]


def test_pair_plan_leaves_odd_one_and_private_sequences_alone():
    lens = [500, 20, 300]
    _, blocks, table = _tables(lens, 0)          # no shared prefix: every first block differs
    assert (pair_plan(table, blocks) == -1).all()
    _, blocks, table = _tables(lens, 64)          # three sharers: (0, 1) paired, 2 alone
    assert pair_plan(table, blocks).tolist() == [1, -2, -1]


@pytest.mark.parametrize("split_blocks", [1, 3, 8, 128, 1024])
def test_loaded_tokens_closed_form_for_shared_prefix(split_blocks):
    # every position of the prefix range is the same block for both sequences
    # of a pair, so each pair saves min(len_a, len_b, prefix) tokens at any split
    rng = np.random.default_rng(11)
    prefix = 2048
    lens = rng.integers(1, 6000, size=20).tolist() + [prefix, 2047, 2049, 16]
    _, blocks, table = _tables(lens, prefix)
    role = pair_plan(table, blocks)
    saved = sum(min(lens[a], lens[b], prefix) for a in range(len(lens))
                for b in [int(role[a])] if b >= 0)
    assert pair_loaded_tokens(table, lens, role, split_blocks) == sum(lens) - saved


def test_loaded_tokens_without_links_is_every_token():
    lens = [700, 100, 333, 288, 1000, 40, 517]
    _, blocks, table = _tables(lens, 288)
    B = len(lens)
    for role in ([-1] * B,
                 [1] + [-1] * (B - 1),                 # one-sided
                 [0] + [-1] * (B - 1),                 # self
                 [B + 3, -2] + [-1] * (B - 2),         # out of range
                 [1, -2 - 5] + [-1] * (B - 2)):        # partner links elsewhere
        assert pair_loaded_tokens(table, lens, np.asarray(role), 4) == sum(lens)


def test_loaded_tokens_split_joint_only_at_equal_first_block():
    # sequence 1 diverges at position 2: with 2-block splits the second split
    # starts on different blocks and is not joint; with 4-block splits it is,
    # and the differing positions are loaded for both sequences
    table = np.array([[0, 1, 2, 3], [0, 1, 5, 6]], dtype=np.int32)
    lens = [64, 60]
    role = np.array([1, -2])
    assert pair_loaded_tokens(table, lens, role, 2) == 32 + 32 + 28
    assert pair_loaded_tokens(table, lens, role, 4) == 32 + 32 + 28
    # reversed roles: sequence 1 is the first of the pair; same loads
    assert pair_loaded_tokens(table, lens, np.array([-3, 0]), 4) == 92
    # the shorter sequence ends inside the shared range
    table = np.array([[0, 1, 2, 3], [0, 1, 2, 7]], dtype=np.int32)
    assert pair_loaded_tokens(table, [64, 40], role, 4) == 64
    assert pair_loaded_tokens(table, [64, 40], role, 1) == 64


def test_loaded_tokens_position_rule():
    # sequence 1 differs from sequence 0 at position 1 only: positions 0, 2 and
    # 3 are loaded once, position 1 once per sequence
    table = np.array([[0, 1, 2, 3], [0, 9, 2, 3]], dtype=np.int32)
    role = np.array([1, -2])
    assert pair_loaded_tokens(table, [64, 64], role, 4) == 16 + 32 + 16 + 16
    # an odd split size: splits [0, 3) and [3, 6), both joint; position 4 differs
    table = np.array([[0, 1, 2, 3, 4, 5], [0, 1, 2, 3, 7, 5]], dtype=np.int32)
    assert pair_loaded_tokens(table, [96, 96], role, 3) == 16 * 3 + (16 + 32 + 16)


def _walk_tokens(table, lens, role, SB):
    """The paired kernel's walk, step by step (joint splits decoded by the first
    sequence of a pair; within one, a position holding the same block in both
    sequences is one load, any other position one load per sequence), summing
    each loaded block's tokens for the sequences it is live for."""
    B = len(lens)
    nb = [(int(n) + 15) // 16 for n in lens]
    total = 0
    for s in range(B):
        o = int(role[s])
        other = o if o >= 0 else -2 - o
        mutual = o != -1 and other != s and 0 <= other < B and (
            (o >= 0 and int(role[other]) == -2 - s) or (o <= -2 and int(role[other]) == s))
        for b0 in range(0, nb[s], SB):
            first, second = (s, other) if o >= 0 else (other, s)
            joint = (mutual and b0 < nb[first] and b0 < nb[second]
                     and table[first][b0] == table[second][b0])
            if joint and s != first:
                continue
            b1a = min(nb[s], b0 + SB)
            if not joint:
                total += sum(min(16, int(lens[s]) - 16 * b) for b in range(b0, b1a))
                continue
            p = second
            b1b = min(nb[p], b0 + SB)
            steps = []
            cur = b0
            while cur < max(b1a, b1b):
                if not (cur < b1a and cur < b1b and table[s][cur] != table[p][cur]):
                    steps.append((cur, 3))
                else:
                    steps += [(cur, 1), (cur, 2)]
                cur += 1
            for q, mask in steps:
                va = min(16, int(lens[s]) - 16 * q) if (mask & 1) and q < b1a else 0
                vb = min(16, int(lens[p]) - 16 * q) if (mask & 2) and q < b1b else 0
                total += max(va, vb)
    return total


@pytest.mark.parametrize("seed", range(6))
def test_loaded_tokens_match_a_step_by_step_walk(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(2, 9))
    lens = [int(x) for x in rng.integers(0, 900, size=B)]
    nbmax = max((n + 15) // 16 for n in lens) + 1
    base = rng.permutation(10_000)[:nbmax]
    table = np.empty((B, nbmax), dtype=np.int64)
    for s in range(B):    # each row copies the base row at random positions
        own = rng.permutation(10_000)[:nbmax] + 10_000 * (s + 1)
        table[s] = np.where(rng.random(nbmax) < 0.6, base, own)
    role = np.full(B, -1)
    order = rng.permutation(B)
    for a_, b_ in zip(order[0::2], order[1::2]):
        if rng.random() < 0.8:
            role[a_], role[b_] = b_, -2 - a_
    for SB in (4, 5, 16):
        assert pair_loaded_tokens(table, lens, role, SB) == _walk_tokens(table, lens, role, SB)
