"""Per-block scoring: normalise, EMA/LRFU, touch, priority, tier (fp64).

Steps, each a plain elementwise definition over the per-(sequence, block)
records:

* normalise: m_hat = mass / max over the sequence's blocks of mass, so the
  hottest block of each sequence scores 1 (the pages leave the scale of the
  EMA input open; this is the reading taken).
* EMA: E <- alpha * m_hat + (1 - alpha) * E, starting from E = 0
  (Visual Reference Sec. 11, Diagram 11.1 update rule; Diagram 11.2's
  worked example starts from 0).  alpha is LRFU's LRU/LFU knob.
* touch: every record of every sequence in the step was read by the
  decode, so its touch count grows by one and its touch timestamp becomes
  the caller's step number (GQA Per-Head Scoring Streams, per-block state:
  touch count and touch timestamp; under dense attention every block of an
  active sequence is read every step, Visual Reference Sec. 4).
* lazy decay: a block that is not touched on a step receives input 0, so
  after a gap of g steps since its last touch its score is
  S_touch * (1 - alpha)^g (RETRACTIONS Sec. 3: the decaying score whose order
  the key K = ln S_touch + t_touch * (-ln(1 - alpha)) preserves).  The update
  at a touch therefore decays the stored score by (1 - alpha)^(step - t_touch);
  for consecutive steps that is the plain one-step EMA.
* eviction candidate: per sequence, the block with the lowest decayed score
  at the current step, ties to the lowest logical block (GQA Per-Head Scoring
  Streams, panel 3: one ordering per sequence, the coldest block is the
  eviction candidate; RETRACTIONS Sec. 3: the victim is audited against a
  brute-force argmin).  Pinned (tier 0) blocks can be excluded.
* priority: P = w_R * R + w_E * E + w_N * N with R = (b + 1) / nb (recency
  of logical block b among the sequence's nb blocks) and N = 1 for anchor
  blocks b < anchor_blocks (Visual Reference Sec. 12, Diagram 12.1:
  0.25 / 0.55 / 0.20).
* tier: 0 (pinned) when P >= t_high, 1 (HBM evictable) when P >= t_low,
  else 2 (CXL) (Visual Reference Sec. 12, Diagram 12.2 cut points 0.3 and
  0.6; Sec. 10 tier names).  Tier 3 is never assigned by P.

A record whose touch timestamp is not older than the new step is left
unchanged and reported (steps must increase).

Parity pins (tests/test_oracle_scoring.py): the printed EMA worked example,
the EMA closed form on constant input, the printed half-life, closed-form
tier sets derived by solving the threshold inequalities, exact cut-point
inclusivity, touch arithmetic, the decay closed form across gaps, and the
printed key's ordering against the decayed score.
"""
from __future__ import annotations

import dataclasses

import numpy as np

NEVER = np.uint64(0xFFFF_FFFF_FFFF_FFFF)
UNCLASSIFIED = np.uint8(0xFF)


@dataclasses.dataclass(frozen=True)
class Policy:
    alpha: float
    w_recency: float = 0.25
    w_ema: float = 0.55
    w_anchor: float = 0.20
    t_low: float = 0.3
    t_high: float = 0.6
    anchor_blocks: int = 1


@dataclasses.dataclass
class ScoreState:
    """One entry per (sequence, logical block), in record order."""
    seq_id: np.ndarray      # uint64, identity key part 1
    block: np.ndarray       # uint64, identity key part 2 (logical block index)
    nblocks: np.ndarray     # int64, blocks of the owning sequence
    seq_index: np.ndarray   # int64, batch slot of the owning sequence
    score: np.ndarray       # float64, EMA E
    t_touch: np.ndarray     # uint64, NEVER before the first touch
    touch_count: np.ndarray  # uint32
    priority: np.ndarray    # float64, last P (0 before the first classify)
    tier: np.ndarray        # uint8, UNCLASSIFIED before the first classify
    anchor: np.ndarray      # bool

    def copy(self) -> "ScoreState":
        return ScoreState(**{f.name: getattr(self, f.name).copy()
                             for f in dataclasses.fields(self)})


def init_state(blocks_per_seq, seq_ids, anchor_blocks: int = 1) -> ScoreState:
    seq_index = np.concatenate([np.full(nb, s, dtype=np.int64)
                                for s, nb in enumerate(blocks_per_seq)])
    block = np.concatenate([np.arange(nb, dtype=np.int64) for nb in blocks_per_seq])
    nblocks = np.concatenate([np.full(nb, nb, dtype=np.int64) for nb in blocks_per_seq])
    n = block.size
    return ScoreState(
        seq_id=np.asarray(seq_ids, dtype=np.uint64)[seq_index],
        block=block.astype(np.uint64),
        nblocks=nblocks,
        seq_index=seq_index,
        score=np.zeros(n, dtype=np.float64),
        t_touch=np.full(n, NEVER, dtype=np.uint64),
        touch_count=np.zeros(n, dtype=np.uint32),
        priority=np.zeros(n, dtype=np.float64),
        tier=np.full(n, UNCLASSIFIED, dtype=np.uint8),
        anchor=block < anchor_blocks,
    )


def normalise(mass_seq):
    """Block mass divided by the sequence's largest block mass."""
    mass_seq = np.asarray(mass_seq, dtype=np.float64)
    if mass_seq.size == 0:      # an empty sequence has no records
        return mass_seq
    top = mass_seq.max()
    if top <= 0.0:
        return np.zeros_like(mass_seq)
    return mass_seq / top


def ema(prev, x, alpha: float):
    """score_t = alpha * x_t + (1 - alpha) * score_{t-1}."""
    return alpha * np.asarray(x, dtype=np.float64) + (1.0 - alpha) * np.asarray(prev, dtype=np.float64)


def recency(block, nblocks):
    return (np.asarray(block, dtype=np.float64) + 1.0) / np.asarray(nblocks, dtype=np.float64)


def priority(score, block, nblocks, anchor, pol: Policy):
    return (pol.w_recency * recency(block, nblocks)
            + pol.w_ema * np.asarray(score, dtype=np.float64)
            + pol.w_anchor * np.asarray(anchor, dtype=np.float64))


def tier_of(p, pol: Policy):
    p = np.asarray(p, dtype=np.float64)
    return np.where(p >= pol.t_high, 0, np.where(p >= pol.t_low, 1, 2)).astype(np.uint8)


def classify(state: ScoreState, pol: Policy) -> ScoreState:
    out = state.copy()
    out.priority = priority(state.score, state.block, state.nblocks, state.anchor, pol)
    out.tier = tier_of(out.priority, pol)
    return out


def score_update(state: ScoreState, masses, step: int, pol: Policy, do_classify: bool = True):
    """One scoring step.  masses: list of per-sequence block-mass arrays.

    Returns (new_state, stale) where stale marks records left unchanged
    because their touch timestamp was not older than `step`.
    """
    out = state.copy()
    m_hat = np.concatenate([normalise(m) for m in masses])
    step_u = np.uint64(step)
    stale = (state.t_touch != NEVER) & (state.t_touch >= step_u)
    upd = ~stale
    prev = decayed(state, step - 1, pol.alpha)   # input 0 on every step since the last touch
    out.score[upd] = ema(prev[upd], m_hat[upd], pol.alpha)
    out.touch_count[upd] = state.touch_count[upd] + np.uint32(1)
    out.t_touch[upd] = step_u
    if do_classify:
        p = priority(out.score, out.block, out.nblocks, out.anchor, pol)
        out.priority[upd] = p[upd]
        out.tier[upd] = tier_of(p, pol)[upd]
    return out, stale


def decayed(state: ScoreState, t: int, alpha: float):
    """Score of every record at step t, given input 0 on the steps after its
    last touch: S_touch * (1 - alpha)^(t - t_touch).  Records never touched
    keep their (zero) score; records touched after t are returned unchanged."""
    touched = state.t_touch != NEVER
    gap = np.zeros(state.score.shape, dtype=np.float64)
    tt = state.t_touch[touched].astype(np.float64)
    gap[touched] = np.maximum(0.0, float(t) - tt)
    return state.score * (1.0 - alpha) ** gap


def order_key(state: ScoreState, alpha: float):
    """The printed order-preserving key K = ln S_touch + t_touch * (-ln(1 - alpha));
    -inf for a zero score."""
    with np.errstate(divide="ignore"):
        k = np.log(state.score) + state.t_touch.astype(np.float64) * (-np.log1p(-alpha))
    return np.where(state.score > 0.0, k, -np.inf)


def eviction_candidates(state: ScoreState, t: int, alpha: float, active=None,
                        exclude_pinned: bool = False, nseq=None):
    """Per sequence, the record with the lowest decayed score at step t (brute
    force over its records; ties to the lowest logical block).  Returns
    (block index or -1, decayed score or +inf) per sequence; inactive
    sequences and sequences with no eligible record give (-1, +inf).  nseq: the
    batch size, when trailing sequences may have no records."""
    s_now = decayed(state, t, alpha)
    if nseq is None:
        nseq = int(state.seq_index.max()) + 1 if state.seq_index.size else 0
    blocks = np.full(nseq, -1, dtype=np.int64)
    scores = np.full(nseq, np.inf)
    for s in range(nseq):
        if active is not None and not active[s]:
            continue
        rows = np.nonzero(state.seq_index == s)[0]
        best = -1
        for r in rows:
            if exclude_pinned and state.tier[r] == 0:
                continue
            if state.t_touch[r] != NEVER and int(state.t_touch[r]) > t:
                continue
            if best < 0 or s_now[r] < s_now[best]:
                best = r
        if best >= 0:
            blocks[s] = int(state.block[best])
            scores[s] = s_now[best]
    return blocks, scores


def grow(state: ScoreState, blocks_per_seq, anchor_blocks: int = 1) -> ScoreState:
    """Records after sequences grew to blocks_per_seq blocks: existing records
    are kept (their sequence's block count, and so their recency, follows the
    new length); each new block gets a fresh record (score 0, never touched,
    unclassified), as a newly allocated block has no history."""
    old_nb = np.zeros(len(blocks_per_seq), dtype=np.int64)
    for s in range(len(blocks_per_seq)):
        old_nb[s] = int((state.seq_index == s).sum())
    seq_ids = np.zeros(len(blocks_per_seq), dtype=np.uint64)
    for s in range(len(blocks_per_seq)):
        rows = np.nonzero(state.seq_index == s)[0]
        if rows.size:
            seq_ids[s] = state.seq_id[rows[0]]
    fresh = init_state(blocks_per_seq, seq_ids, anchor_blocks)
    out = fresh.copy()
    for s in range(len(blocks_per_seq)):
        if blocks_per_seq[s] < old_nb[s]:
            raise ValueError("sequences only grow")
        src = np.nonzero(state.seq_index == s)[0]
        dst = np.nonzero(fresh.seq_index == s)[0][: src.size]
        for f in ("seq_id", "block", "score", "t_touch", "touch_count", "priority", "tier",
                  "anchor"):
            getattr(out, f)[dst] = getattr(state, f)[src]
    return out
