"""GPU: seeded random small problems across the three stored formats, split
sizes, layer ranges, shared prefixes and pairings, each against the oracle
(attention outputs of the layers in range and block mass), and the paired
decode's bits against the unpaired decode's.  Lengths mix random values with
the boundary cases (0, 1, block edges, the KIVI residual window's edges)."""
import math

import numpy as np
import pytest
import torch

import workload as W
from oracle import kivi as KV
from paged_gqa_kv_amd.session import DecodeSession

from . import parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda"
SCALE = 1.0 / math.sqrt(128.0)
EDGES = [0, 1, 15, 16, 17, 31, 32, 33, 159, 160, 161, 191, 192, 255, 256, 257]
FORMATS = ["fp16", "e4m3", "kivi2"]


def _params(k):
    rng = np.random.default_rng(4242 + k)
    fmt = FORMATS[k % 3]
    L = int(rng.integers(1, 4))
    B = int(rng.integers(1, 7))
    lens = [int(rng.choice(EDGES)) if rng.random() < 0.45 else int(rng.integers(1, 1300))
            for _ in range(B)]
    if max(lens) == 0:
        lens[int(rng.integers(B))] = int(rng.integers(1, 400))
    shared = int(rng.choice([0, 0, 16, 48, 160, 300]))
    sb = int(rng.choice([0, 4, 6, 8, 12, 32]))
    lb = int(rng.integers(0, L))
    le = int(rng.integers(lb + 1, L + 1))
    pair = fmt != "kivi2" and shared > 0 and bool(rng.random() < 0.75)
    seed = int(rng.integers(1, 1 << 30))
    return fmt, L, lens, shared, sb, lb, le, pair, seed


@pytest.mark.parametrize("k", range(40))
def test_random_problem_against_oracle(k):
    fmt, L, lens, shared, sb, lb, le, pair, seed = _params(k)
    print(f"\n[case] random #{k}: {fmt}, {L} layers, lens {lens}, shared {shared}, "
          f"split {sb}, layers [{lb}, {le}), paired {pair}, seed {seed}", flush=True)
    wl = W.custom(f"rand{k}", L, lens, seed=seed, spare_blocks=5, shared_prefix_tokens=shared)
    if fmt == "e4m3":
        wl = W.as_e4m3(wl)
    elif fmt == "kivi2":
        wl = W.as_kivi2(wl)
    m = W.materialise(wl, DEV)
    sess = DecodeSession(m, layer_begin=lb, layer_end=le, split_blocks=sb,
                         pair_role="auto" if pair else None)
    q = W.make_query(m, k)
    sess.decode(q)
    torch.cuda.synchronize()
    assert sess.status() == 0
    qh = q.cpu().numpy()
    if fmt == "kivi2":
        out_ref, mass_ref = KV.decode_step(qh, m.pool.cpu().numpy(), m.table_host, m.lens, SCALE,
                                           lb, le)
    else:
        out_ref, mass_ref = P.oracle_decode(P.host(m), qh, lb, le)
    live = [s for s in range(m.batch) if m.lens[s] > 0]
    P.check_out(sess.out, out_ref, range(lb, le), seqs=live)
    P.check_mass(sess.mass, mass_ref, m.meta_offsets.cpu().numpy(), seqs=live)
    out = sess.out.float().cpu().numpy()
    for s in range(m.batch):
        if m.lens[s] == 0:
            assert not out[s, lb:le].any(), s
    if pair:
        ref = DecodeSession(m, layer_begin=lb, layer_end=le, split_blocks=sess.split_blocks)
        ref.decode(q)
        torch.cuda.synchronize()
        assert torch.equal(ref.out.view(torch.int16), sess.out.view(torch.int16))
        assert torch.equal(ref.mass.view(torch.int32), sess.mass.view(torch.int32))
