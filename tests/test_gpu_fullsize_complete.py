"""Full-size checks that leave nothing to sampling.

* One complete decode step of the 128K-token, 80-layer workload against the
  oracle: all 5,120 (layer, head) output rows, all 8,192 block masses from the
  oracle's own decode, and the scoring of every record driven by the oracle's
  mass (alpha 0.05 and 0.15); the same for its E4M3 and KIVI forms, the
  32-sequence shared-prefix batch and the 1M-token, 32-layer sequence.  The
  oracle runs per (sequence, layer) on host threads (oracle/runner.py) over
  the layer's blocks copied from the device.
  This is the aggregation of the 640 (layer, KV-head) streams into one score
  per block ("GQA Per-Head Scoring Streams", panel 2) at its real size.
* The closed-form tier table at the configs' shapes, run through the GPU: with
  q = 0 every logit is 0, so each head attends uniformly, every full block's
  mass is exactly 16 L 64 / n and its normalised mass is 1; after S steps
  E = 1 - (1 - alpha)^S and every label follows from
  P = 0.25 (b + 1) / nb + 0.55 E + 0.20 [b = 0] and the cut points 0.3 / 0.6
  ("Visual Reference" Sec. 11, Diagram 11.1; Sec. 12, Diagrams 12.1-12.2).
  The nearest priority sits 1.7e-6 from a cut point, far above rounding, so
  every label must match, the ones inside the 1e-4 band included.
"""
import math

import numpy as np
import pytest
import torch

import workload as W
from oracle import runner as OR
from oracle import scoring as OS
from paged_gqa_kv_amd import api
from paged_gqa_kv_amd.session import DecodeSession

from . import parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda"
SCALE = 1.0 / math.sqrt(128.0)


def _case(msg):
    print(f"\n[case] {msg}", flush=True)


def _host_layer(m, s, layer):
    nb = m.blocks[s]
    pids = m.block_table[s, :nb].long()
    return m.pool[pids, layer].cpu().numpy()[:, None]          # [nb][1][2][8][16][128]


@pytest.fixture(scope="module")
def m128k():
    m = W.materialise(W.WORKLOADS["decode-80L-128K"], DEV)
    torch.cuda.synchronize()
    yield m
    del m
    torch.cuda.empty_cache()


def _complete_step(m, name, threads=None, blas_threads=2):
    """One decode step (step 0's query) of materialised workload m on the GPU,
    in the launch configuration bench.py times, against the oracle: every
    output row, every block mass, and the scoring of every record driven by
    the oracle's mass, for each of the workload's alphas."""
    fmt = m.workload.kv_format
    L = m.num_layers
    _case(f"{name} ({fmt} KV), step 0: every output row, every block mass, every record")
    sess = DecodeSession(m)
    q = W.make_query(m, 0)
    sess.decode(q)
    torch.cuda.synchronize()
    assert sess.status() == 0
    out_ref, mass_ref, info = OR.decode_layers(
        q.cpu().numpy(), lambda s, layer: _host_layer(m, s, layer), m.lens, range(L), SCALE,
        kv_format=fmt, threads=threads, blas_threads=blas_threads,
        progress=lambda msg: print("  " + msg, flush=True) if msg.endswith("79 done") or
        L < 80 else None)
    print(f"  oracle: {info['wall_s']:.1f} s on {info['workers']} threads x "
          f"{info['blas_threads']} BLAS threads ({info['fetch_s']:.1f} s of it in copies)",
          flush=True)
    assert not np.isnan(out_ref).any()
    w_out = P.check_out(sess.out, out_ref, range(L))
    offsets = m.meta_offsets.cpu().numpy()
    w_mass = P.check_mass(sess.mass, mass_ref, offsets)
    print(f"  all {m.batch * L * 64} rows: worst {w_out:.2e} of the row maximum; all "
          f"{m.total_blocks} masses: worst relative {w_mass:.2e}", flush=True)
    for alpha in m.workload.alphas:
        pol = OS.Policy(alpha=alpha)
        sess.reset_meta()
        sess.score(0, api.policy(alpha))
        state = OS.init_state(m.blocks, m.seq_ids.cpu().numpy())
        state, stale = OS.score_update(state, mass_ref, 0, pol)
        assert not stale.any()
        err, near = P.check_records(sess.records(), state, pol)
        print(f"  alpha {alpha}: all {m.total_blocks} records, max |dE| {err:.2e}, {near} "
              f"labels in the cut-point band", flush=True)
    assert sess.status() == 0
    del sess


def test_fullsize_128k_complete_step_against_the_oracle(m128k):
    _complete_step(m128k, "decode-80L-128K")


@pytest.mark.parametrize("name,fmt,threads,blas", [
    ("decode-80L-128K", "e4m3", None, 2),
    ("decode-80L-128K", "kivi2", None, 2),
    ("decode-80L-32xMixed-shared2K", "fp16", None, 1),
])
def test_fullsize_complete_step_against_the_oracle(name, fmt, threads, blas):
    wl = W.WORKLOADS[name]
    if fmt == "e4m3":
        wl = W.as_e4m3(wl)
    elif fmt == "kivi2":
        wl = W.as_kivi2(wl)
    m = W.materialise(wl, DEV)
    torch.cuda.synchronize()
    _complete_step(m, name, threads=threads, blas_threads=blas)
    del m
    torch.cuda.empty_cache()


def _closed_form(nb, alpha, steps):
    E = 1.0 - (1.0 - alpha) ** steps
    b = np.arange(nb)
    p = 0.25 * (b + 1) / nb + 0.55 * E + 0.20 * (b == 0)
    tier = np.where(p >= 0.6, 0, np.where(p >= 0.3, 1, 2)).astype(np.uint8)
    band = (np.abs(p - 0.3) < 1e-4) | (np.abs(p - 0.6) < 1e-4)
    return E, p, tier, band


def _run_q0(m, alpha, steps, counts, band_count):
    L, n, nb = m.num_layers, m.lens[0], m.blocks[0]
    sess = DecodeSession(m)
    q = torch.zeros((1, L, 64, 128), dtype=torch.float16, device=DEV)
    for step in range(steps):
        sess.step(q, step, api.policy(alpha))
        if step == 0:
            mass = sess.mass[:nb].cpu().numpy()
            # every logit 0: each (layer, head) puts 16 / n on a full block
            assert np.all(mass == np.float32(16.0 * L * 64 / n)), np.unique(mass)[:5]
    torch.cuda.synchronize()
    assert sess.status() == 0
    E, p, tier, band = _closed_form(nb, alpha, steps)
    rec = sess.records()
    assert np.abs(rec["score"] - E).max() <= 1e-12
    assert np.abs(rec["priority"] - p).max() <= 1e-12
    assert np.all(rec["touch_count"] == steps)
    assert np.all(rec["t_touch"] == steps - 1)
    assert np.array_equal(rec["tier"], tier), np.nonzero(rec["tier"] != tier)[0][:10]
    got = [int((rec["tier"] == k).sum()) for k in range(3)]
    assert got == counts == [int((tier == k).sum()) for k in range(3)]
    assert int(band.sum()) == band_count
    print(f"  alpha {alpha}, {steps} steps: E = {E:.6f}, tiers {got}, {band_count} labels "
          f"within 1e-4 of a cut point, all equal to the closed form", flush=True)


@pytest.mark.parametrize("alpha,counts,band", [(0.05, [0, 8192, 0], 0),
                                               (0.15, [5217, 2975, 0], 6)])
def test_fullsize_128k_closed_form_tiers(m128k, alpha, counts, band):
    _case(f"decode-80L-128K with q = 0, alpha {alpha}, 16 steps: closed-form labels")
    _run_q0(m128k, alpha, 16, counts, band)


@pytest.fixture(scope="module")
def m1m():
    m = W.materialise(W.WORKLOADS["decode-32L-1M"], DEV)
    torch.cuda.synchronize()
    yield m
    del m
    torch.cuda.empty_cache()


def test_fullsize_1m_complete_step_against_the_oracle(m1m):
    # 1M tokens: 17 GB of fp64 keys and values per piece, so 4 pieces at a time
    _complete_step(m1m, "decode-32L-1M", threads=16, blas_threads=4)


@pytest.mark.parametrize("alpha,counts,band", [(0.01, [0, 0, 65536], 0),
                                               (0.15, [0, 55811, 9725], 52)])
def test_fullsize_1m_closed_form_tiers(m1m, alpha, counts, band):
    _case(f"decode-32L-1M with q = 0, alpha {alpha}, 4 steps: closed-form labels")
    _run_q0(m1m, alpha, 4, counts, band)
