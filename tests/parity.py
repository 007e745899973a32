"""Comparison helpers for the GPU-vs-oracle parity tests.

Tolerances (the bar every GPU test applies):
  * attention output: per (sequence, layer, head) row,
    max_d |gpu - ref| <= 2e-3 * max_d |ref|;
  * block mass: |gpu - ref| <= 1e-5 * ref + 1e-7 * max(ref) (fp32 logits and
    exponentials against fp64; derived in the design notes);
  * EMA score: |gpu - ref| <= 1e-5 absolute;
  * touch count and timestamp: bit-exact;
  * tier: exact, except records whose oracle priority lies within 1e-4 of a
    cut point; priority within 1e-5.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from oracle import attention as OA
from oracle import scoring as OS

OUT_RTOL = 2e-3
MASS_RTOL = 1e-5
SCORE_ATOL = 1e-5
TIER_BAND = 1e-4
SCALE = 1.0 / math.sqrt(128.0)


def host(m):
    """Host copies of a materialised workload, for the oracle."""
    return dict(pool=m.pool.cpu().numpy(), table=m.table_host, lens=list(m.lens),
                kv_format=m.workload.kv_format)


def oracle_decode(h, q, layer_begin=0, layer_end=None):
    qn = q.cpu().numpy() if isinstance(q, torch.Tensor) else q
    return OA.decode_step(qn, h["pool"], h["table"], h["lens"], SCALE, layer_begin, layer_end,
                          kv_format=h.get("kv_format", "fp16"))


def check_out(gpu_out, ref_out, layers, seqs=None):
    g = gpu_out.float().cpu().numpy().astype(np.float64)
    seqs = range(ref_out.shape[0]) if seqs is None else seqs
    worst = 0.0
    for s in seqs:
        for layer in layers:
            ref = ref_out[s, layer]
            err = np.abs(g[s, layer] - ref).max(axis=1)
            lim = np.abs(ref).max(axis=1)
            ratio = float((err / np.maximum(lim, 1e-30)).max())
            worst = max(worst, ratio)
            assert np.all(err <= OUT_RTOL * lim), (s, layer, ratio)
    return worst


def check_mass(gpu_mass, ref_masses, offsets, seqs=None):
    g = gpu_mass.cpu().numpy().astype(np.float64)
    seqs = range(len(ref_masses)) if seqs is None else seqs
    worst = 0.0
    for s in seqs:
        ref = ref_masses[s]
        got = g[offsets[s]:offsets[s] + ref.size]
        err = np.abs(got - ref)
        tol = MASS_RTOL * ref + 1e-7 * ref.max()
        assert np.all(err <= tol), (s, float((err / ref).max()))
        worst = max(worst, float((err / ref).max()))
    return worst


def check_records(rec, state: OS.ScoreState, pol: OS.Policy, rows=None):
    """rec: numpy META_DTYPE records; state: oracle state (same record order)."""
    idx = np.arange(len(state.score)) if rows is None else np.asarray(rows)
    r = rec[idx]
    assert np.array_equal(r["key"][:, 0], state.seq_id[idx])
    assert np.array_equal(r["key"][:, 1], state.block[idx])
    assert np.array_equal(r["touch_count"], state.touch_count[idx])
    assert np.array_equal(r["t_touch"], state.t_touch[idx])
    assert np.array_equal((r["flags"] & 1).astype(bool), state.anchor[idx])
    err = np.abs(r["score"] - state.score[idx])
    assert err.max(initial=0.0) <= SCORE_ATOL, float(err.max())
    classified = state.tier[idx] != OS.UNCLASSIFIED
    assert np.array_equal(r["tier"] == 0xFF, ~classified)
    p = state.priority[idx]
    perr = np.abs(r["priority"] - p)[classified]
    assert perr.max(initial=0.0) <= SCORE_ATOL
    near = (np.abs(p - pol.t_low) < TIER_BAND) | (np.abs(p - pol.t_high) < TIER_BAND)
    must = classified & ~near
    assert np.array_equal(r["tier"][must], state.tier[idx][must])
    return float(err.max(initial=0.0)), int(near[classified].sum())
