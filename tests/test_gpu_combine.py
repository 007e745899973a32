"""GPU: the one-launch split combine and mass reduction (combine_mass) on both
of its weight paths.  A mass work-group takes a row's split statistics into
registers when the sequence has at most 16 splits and walks them in a loop
otherwise; both must give the oracle's output and block mass, also when one
launch mixes sequences of both kinds."""
import math

import pytest
import torch

import workload as W
from paged_gqa_kv_amd.session import DecodeSession

from . import parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda"
FUSED_MAX_WEIGHTS = 4096           # (layer, head) rows x splits the one-launch form holds
FUSED_MAX_STAT_BYTES = 2 << 20     # statistics all its mass work-groups re-read
REGISTER_SPLITS = 16


def _case(msg):
    print(f"\n[case] {msg}", flush=True)


def _one_launch(max_nb, batch, layers, split):
    """Whether a batch takes the one-launch form (the sizes it is chosen by:
    the block table's width, the batch, the layers and the split)."""
    n_splits = -(-max_nb // split)
    weights = layers * 64 * n_splits
    col_groups = -(-max_nb // 32)
    return weights <= FUSED_MAX_WEIGHTS and weights * 8 * col_groups * batch <= FUSED_MAX_STAT_BYTES


@pytest.mark.parametrize("lens,split,paths", [
    ([400 * 16], 16, {"loop"}),                       # 25 splits
    ([400 * 16], 32, {"registers"}),                  # 13 splits
    ([400 * 16, 17 * 16 + 5, 3, 256 * 16 + 1], 16, {"loop", "registers"}),
])
def test_one_launch_combine_both_weight_paths(lens, split, paths):
    _case(f"combine_mass, 1 layer, lengths {lens}, split_blocks={split}, paths {sorted(paths)}")
    m = W.materialise(W.custom("comb", 1, lens, seed=41, spare_blocks=5), DEV)
    assert _one_launch(m.table_host.shape[1], len(lens), 1, split)
    nsp = [math.ceil(math.ceil(n / 16) / split) for n in lens]
    assert {"registers" if k <= REGISTER_SPLITS else "loop" for k in nsp} == paths
    sess = DecodeSession(m, split_blocks=split)
    assert sess.split_blocks == split
    q = W.make_query(m, 0)
    sess.decode(q)
    torch.cuda.synchronize()
    out_ref, mass_ref = P.oracle_decode(P.host(m), q)
    P.check_out(sess.out, out_ref, range(m.num_layers))
    P.check_mass(sess.mass, mass_ref, m.meta_offsets.cpu().numpy())
    assert sess.status() == 0
