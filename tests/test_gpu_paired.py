"""GPU: the paired decode (kvs_decode_step_paired over fp16,
kvs_decode_step_e4m3_paired over E4M3), where one wave serves two sequences
that share blocks, gives the unpaired decode's bits and the oracle's values,
whatever the pairing array holds."""
import numpy as np
import pytest
import torch

import workload as W
from paged_gqa_kv_amd import api
from paged_gqa_kv_amd.session import DecodeSession, pair_plan

from . import parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _case(msg):
    print(f"\n[case] {msg}", flush=True)


def _bits(t):
    return t.contiguous().view(torch.int16 if t.dtype == torch.float16 else torch.int32)


FORMATS = ["fp16", "e4m3"]


def _fmt(wl, fmt):
    return W.as_e4m3(wl) if fmt == "e4m3" else wl


def _shared_workload(seed=9, layers=2, fmt="fp16"):
    # an 18-block (288-token) shared prefix; 100 and 40 tokens are shorter than
    # it, so their last shared block is partial for them and full for others
    lens = [700, 100, 333, 288, 1000, 40, 517]
    return W.materialise(_fmt(W.custom("pair", layers, lens, seed=seed, spare_blocks=6,
                                       shared_prefix_tokens=288), fmt), DEV)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("split_blocks", [4, 5, 8, 0])
def test_paired_decode_bits_and_oracle(split_blocks, fmt):
    _case(f"{fmt} paired vs unpaired decode, shared 288-token prefix, split_blocks={split_blocks}")
    m = _shared_workload(fmt=fmt)
    role = pair_plan(m.table_host, m.blocks)
    assert (role >= 0).sum() == 3 and (role <= -2).sum() == 3
    par = DecodeSession(m, split_blocks=split_blocks, pair_role=role)
    assert par.split_blocks <= 512
    ref = DecodeSession(m, split_blocks=par.split_blocks)
    h = P.host(m)
    offs = m.meta_offsets.cpu().numpy()
    for step in range(2):
        q = W.make_query(m, step)
        ref.decode(q)
        par.decode(q)
        torch.cuda.synchronize()
        assert torch.equal(_bits(par.out), _bits(ref.out)), step
        assert torch.equal(_bits(par.mass), _bits(ref.mass)), step
        out_ref, mass_ref = P.oracle_decode(h, q)
        P.check_out(par.out, out_ref, range(m.num_layers))
        P.check_mass(par.mass, mass_ref, offs)
    assert par.status() == 0 and ref.status() == 0


def _check_pairing(m, role, split_blocks, step=0):
    par = DecodeSession(m, split_blocks=split_blocks, pair_role=np.asarray(role, dtype=np.int32))
    ref = DecodeSession(m, split_blocks=split_blocks)
    q = W.make_query(m, step)
    ref.decode(q)
    par.decode(q)
    torch.cuda.synchronize()
    assert torch.equal(_bits(par.out), _bits(ref.out))
    assert torch.equal(_bits(par.mass), _bits(ref.mass))
    out_ref, mass_ref = P.oracle_decode(P.host(m), q)
    P.check_out(par.out, out_ref, range(m.num_layers))
    P.check_mass(par.mass, mass_ref, m.meta_offsets.cpu().numpy())
    assert par.status() == 0 and ref.status() == 0


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("split_blocks", [4, 16])
def test_paired_decode_first_sequence_shorter(split_blocks, fmt):
    _case(f"{fmt} pairs whose first sequence is the shorter one, split_blocks={split_blocks}")
    m = _shared_workload(seed=4, fmt=fmt)
    # reverse every link of the shared-prefix plan: the second sequence of each
    # pair becomes the first, so joint splits run past the first one's end
    plan = pair_plan(m.table_host, m.blocks)
    role = np.full(m.batch, -1, dtype=np.int32)
    for a_, b_ in ((a_, int(plan[a_])) for a_ in range(m.batch) if plan[a_] >= 0):
        role[b_] = a_
        role[a_] = -2 - b_
    _check_pairing(m, role, split_blocks)


@pytest.mark.parametrize("fmt", FORMATS)
def test_paired_decode_shared_blocks_between_private_ones(fmt):
    _case(f"{fmt} pairs sharing blocks at some positions only (shared, private, shared again)")
    m = W.materialise(_fmt(W.custom("mix", 2, [300, 250, 180, 400], seed=21, spare_blocks=4),
                           fmt), DEV)
    # make sequence 1 share sequence 0's blocks at positions 0-3 and 8-11 (4-7
    # stay its own), and sequence 3 share sequence 2's blocks at positions 4-7
    # and 9 (not at 0-3 or 8); the tables on both sides of the boundary change
    # together.  Splits of 4 then have joint splits after private ones, and a
    # shared position inside a split that is not joint.
    t = m.table_host
    for b in (0, 1, 2, 3, 8, 9, 10, 11):
        t[1, b] = t[0, b]
    for b in (4, 5, 6, 7, 9):
        t[3, b] = t[2, b]
    m.block_table.copy_(torch.from_numpy(t).to(DEV))
    role = [1, -2, 3, -4]
    for sb in (4, 5, 8, 16):
        _check_pairing(m, role, sb)


@pytest.mark.parametrize("fmt", FORMATS)
def test_inconsistent_pair_roles_change_nothing(fmt):
    _case(f"{fmt} pair_role arrays with broken, one-sided, self and out-of-range links")
    m = _shared_workload(seed=3, fmt=fmt)
    B = m.batch
    ref = DecodeSession(m, split_blocks=8)
    q = W.make_query(m, 0)
    ref.decode(q)
    torch.cuda.synchronize()
    roles = {
        "one-sided": [1] + [-1] * (B - 1),
        "links elsewhere": [1, -2 - 5] + [-1] * (B - 2),
        "self": [0] + [-1] * (B - 1),
        "out of range": [B + 3, -2 - 0] + [-1] * (B - 2),
        "negative partner": [-2 - (B + 7)] + [-1] * (B - 1),
        "second below first": [-3, 0] + [-1] * (B - 2),      # pair (1, 0)
        "all unpaired": [-1] * B,
        "everyone with 0": [3] + [-2 - 0] * (B - 1),          # 0 -> 3 linked; the others point at 0
    }
    for name, role in roles.items():
        par = DecodeSession(m, split_blocks=8, pair_role=np.asarray(role, dtype=np.int32))
        par.decode(q)
        torch.cuda.synchronize()
        assert torch.equal(_bits(par.out), _bits(ref.out)), name
        assert torch.equal(_bits(par.mass), _bits(ref.mass)), name
        assert par.status() == 0, name


@pytest.mark.parametrize("fmt", FORMATS)
def test_pairs_without_shared_blocks(fmt):
    _case(f"{fmt} pairs whose sequences share no block: every split decoded separately")
    m = W.materialise(_fmt(W.custom("nopair", 2, [300, 517, 64, 1], seed=12, spare_blocks=4),
                           fmt), DEV)
    ref = DecodeSession(m, split_blocks=4)
    par = DecodeSession(m, split_blocks=4, pair_role=np.asarray([1, -2, 3, -4], dtype=np.int32))
    q = W.make_query(m, 1)
    ref.decode(q)
    par.decode(q)
    torch.cuda.synchronize()
    assert torch.equal(_bits(par.out), _bits(ref.out))
    assert torch.equal(_bits(par.mass), _bits(ref.mass))


def test_paired_decode_rejects_before_launch():
    _case("paired entry point: NULL pair_role, split above 512, KIVI session")
    m = _shared_workload(seed=5)
    sess = DecodeSession(m, split_blocks=8, pair_role="auto")
    with pytest.raises(api.KvsError):
        api.decode_step_paired(sess.shape, W.make_query(m, 0), m.pool, m.pool_blocks,
                               m.block_table, m.max_blocks, m.seq_lens, None, m.meta_offsets,
                               m.batch, m.total_blocks, 0, m.num_layers, api.DEFAULT_SCALE,
                               sess.out, sess.mass, 0, 8, sess.ws)
    with pytest.raises(api.KvsError):
        api.decode_step_paired(sess.shape, W.make_query(m, 0), m.pool, m.pool_blocks,
                               m.block_table, m.max_blocks, m.seq_lens, sess.pair_role,
                               m.meta_offsets, m.batch, m.total_blocks, 0, m.num_layers,
                               api.DEFAULT_SCALE, sess.out, sess.mass, 0, 1024, sess.ws)
    with pytest.raises(ValueError):
        DecodeSession(W.materialise(W.as_kivi2(W.WORKLOADS["decode-1L-1K"]), DEV),
                      pair_role="auto")
    e4 = _shared_workload(seed=5, fmt="e4m3")
    sess = DecodeSession(e4, split_blocks=8, pair_role="auto")
    with pytest.raises(api.KvsError):
        api.decode_step_e4m3_paired(sess.shape, W.make_query(e4, 0), e4.pool, e4.pool_blocks,
                                    e4.block_table, e4.max_blocks, e4.seq_lens, None,
                                    e4.meta_offsets, e4.batch, e4.total_blocks, 0,
                                    e4.num_layers, api.DEFAULT_SCALE, sess.out, sess.mass, 0, 8,
                                    sess.ws)


@pytest.mark.parametrize("split_blocks", [16, 5, 37])
@pytest.mark.parametrize("fmt", FORMATS)
def test_two_heads_per_wave_decode_matches_one_head_per_wave_bit_for_bit(fmt, split_blocks):
    """Sequences that fill their splits: the fp16 decode then serves two KV heads
    per wave (records >= 3/4 of batch x splits x split blocks), as the E4M3
    decode always does.  The paired decode with no pairs serves one head per
    wave; per query head the arithmetic is the same, so every bit must match,
    and both match the oracle."""
    _case(f"{fmt}: 4 x 1,024 tokens at split {split_blocks} (two heads per wave) against the "
          "paired decode with no pairs (one head per wave)")
    m = W.materialise(_fmt(W.custom("full", 2, [1024, 1024, 1024, 1000], seed=31,
                                    spare_blocks=3), fmt), DEV)
    n_splits = -(-64 // split_blocks)
    assert 4 * m.total_blocks >= 3 * m.batch * n_splits * split_blocks   # the two-heads rule holds
    q = W.make_query(m, 0)
    one = DecodeSession(m, split_blocks=split_blocks,
                        pair_role=np.full(m.batch, -1, dtype=np.int32))
    two = DecodeSession(m, split_blocks=split_blocks)
    one.decode(q)
    two.decode(q)
    torch.cuda.synchronize()
    assert one.status() == 0 and two.status() == 0
    assert torch.equal(_bits(one.out), _bits(two.out))
    assert torch.equal(_bits(one.mass), _bits(two.mass))
    out_ref, mass_ref = P.oracle_decode(P.host(m), q)
    P.check_out(two.out, out_ref, range(m.num_layers))
    P.check_mass(two.mass, mass_ref, m.meta_offsets.cpu().numpy())
