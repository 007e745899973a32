"""GPU parity of the FP8 E4M3 decode (kvs_decode_step_e4m3) against the oracle
decoding the same codes exactly."""
import numpy as np
import pytest
import torch

import workload as W
from paged_gqa_kv_amd import api
from paged_gqa_kv_amd.session import DecodeSession

from . import parity as P
from .test_gpu_parity import _run_pipeline

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _case(msg):
    print(f"\n[case] {msg}", flush=True)


# The E4M3 decode serves two KV heads per wave; splits that are not multiples
# of 4 round its LDS block-id list up and pad its mass-partial rows, and 1,024
# blocks need 74 KB of LDS (above 64 KiB).
@pytest.mark.parametrize("split_blocks", [4, 5, 7, 16, 37, 64, 1024])
def test_e4m3_ragged_batch(split_blocks):
    _case(f"E4M3 KV, ragged lengths, 2 layers, split_blocks={split_blocks}")
    wl = W.custom("ragged8", 2, [1, 15, 16, 17, 37, 300, 1000, 2049], seed=41, spare_blocks=9,
                  kv_format="e4m3")
    m = W.materialise(wl, DEV)
    assert m.pool.dtype == torch.uint8
    _run_pipeline(m, 0.05, 3, split_blocks=split_blocks)


def test_e4m3_tiny_workload_and_poisoned_spares():
    _case("E4M3 KV, 1 layer x 1,024 tokens, 10 steps; spare blocks hold the NaN code")
    m = W.materialise(W.as_e4m3(W.WORKLOADS["decode-1L-1K"]), DEV)
    used = np.zeros(m.pool_blocks, bool)
    used[m.table_host[m.table_host >= 0]] = True
    assert (m.pool[torch.from_numpy(np.nonzero(~used)[0]).to(DEV)] == 0x7F).all()
    sess, _ = _run_pipeline(m, 0.15, 10)
    assert torch.isfinite(sess.out).all()


def test_e4m3_4L_8x8K_workload():
    _case("E4M3 KV, decode-4L-8x8K, 6 steps; decode parity on all sequences at steps 0 and 5")
    m = W.materialise(W.as_e4m3(W.WORKLOADS["decode-4L-8x8K"]), DEV)
    _run_pipeline(m, 0.15, 6, check_decode_steps={0, 5}, score_seqs=[2])


def test_e4m3_permutation_bit_invariance():
    _case("E4M3 KV, physical permutation leaves every bit unchanged")
    wl = W.custom("perm8", 2, [700, 64, 333], seed=5, spare_blocks=20, kv_format="e4m3")
    m = W.materialise(wl, DEV)
    q = W.make_query(m, 0)
    s1 = DecodeSession(m, split_blocks=16)
    s1.decode(q)
    perm = torch.randperm(m.pool_blocks, generator=torch.Generator().manual_seed(2)).to(DEV)
    pool2 = torch.empty_like(m.pool)
    pool2[perm] = m.pool
    table2 = torch.where(m.block_table >= 0, perm[m.block_table.clamp(min=0).long()].int(),
                         m.block_table)
    m2 = type(m)(**{**m.__dict__, "pool": pool2, "block_table": table2})
    s2 = DecodeSession(m2, split_blocks=16)
    s2.decode(q)
    torch.cuda.synchronize()
    assert torch.equal(s1.out.view(torch.int16), s2.out.view(torch.int16))
    assert torch.equal(s1.mass.view(torch.int32), s2.mass.view(torch.int32))


def test_e4m3_nan_value_reaches_the_other_head_of_its_pair_only():
    """A wave serves KV heads 2i and 2i + 1.  A NaN code among head 3's values
    makes that channel NaN in the output rows of heads 3 and 2 (query heads
    16-31), as documented for kvs_decode_step_e4m3; every other element matches
    the oracle, and the block mass (from the keys) is untouched."""
    _case("E4M3 KV, one NaN value code in KV head 3 of sequence 0: pair-wide NaN, nothing else")
    wl = W.custom("nanpair", 1, [100, 40], seed=13, spare_blocks=3, kv_format="e4m3")
    m = W.materialise(wl, DEV)
    pid = int(m.table_host[0, 2])
    token, chan = 5, 77                      # token 32 + 5 of sequence 0, value channel 77
    m.pool[pid, 0, 1, 3, token, chan] = 0x7F
    torch.cuda.synchronize()
    q = W.make_query(m, 0)
    sess = DecodeSession(m, split_blocks=4)
    sess.decode(q)
    torch.cuda.synchronize()
    out = sess.out.float().cpu().numpy().astype(np.float64)
    out_ref, mass_ref = P.oracle_decode(P.host(m), q)
    nan = np.isnan(out)
    expect = np.zeros_like(nan)
    expect[0, 0, 16:32, chan] = True
    assert np.array_equal(nan, expect), np.argwhere(nan != expect)[:5]
    assert np.isnan(out_ref[0, 0, 24:32, chan]).all() and not np.isnan(out_ref[0, 0, 16:24]).any()
    # every other element to the usual bar: 2e-3 of its row's largest element
    a = np.where(expect, 0.0, out)
    r = np.where(expect, 0.0, out_ref)
    err = np.abs(a - r).max(axis=-1)
    lim = np.abs(r).max(axis=-1)
    assert np.all(err <= P.OUT_RTOL * lim), float((err / np.maximum(lim, 1e-30)).max())
    P.check_mass(sess.mass, mass_ref, m.meta_offsets.cpu().numpy())
