"""GPU: the bandwidth probe (kvs_stream_probe) reads every 16-byte word of the
buffer exactly once (the XOR of its per-lane words equals the XOR of the
buffer) and copies exactly, for sizes with a ragged tail and several grids."""
import numpy as np
import pytest
import torch

from paged_gqa_kv_amd import api

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 8192 + 48, (1 << 20) + 16 * 37, 3 << 22])
@pytest.mark.parametrize("grid", [0, 1, 3, 100])
def test_stream_probe_reads_everything_once_and_copies(nbytes, grid):
    print(f"\n[case] stream probe, {nbytes} bytes, grid {grid}", flush=True)
    g = torch.Generator().manual_seed(nbytes + grid)
    src = torch.randint(0, 2**31 - 1, (nbytes // 4,), generator=g, dtype=torch.int32).cuda()
    groups = grid if grid else 2048
    sink = torch.zeros(groups * 256, dtype=torch.int32, device="cuda")
    api.stream_probe(src, sink, nbytes, 0, grid)
    dst = torch.zeros_like(src)
    api.stream_probe(src, dst, nbytes, 1, grid)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(src.cpu().numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want
    assert torch.equal(dst, src)
