"""The C-ABI library loads, exports what include/kvs.h declares, and rejects
every host-checkable bad argument before launching anything (no GPU needed:
none of these calls reaches the device)."""
import ctypes
import os
import re

import pytest

from paged_gqa_kv_amd import _abi, api
from paged_gqa_kv_amd._abi import (KVS_E_ALIGN, KVS_E_NULL, KVS_E_POLICY, KVS_E_RANGE,
                                   KVS_E_SHAPE, KVS_E_WORKSPACE, KvsError)
from oracle import arithmetic as A

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "kvs.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"\b(kvs_[a-z0-9_]+)\s*\(", src))


def test_every_declared_function_is_exported():
    lib = _abi.lib()
    declared = _declared()
    assert declared == set(_abi.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_byte_accounting_matches_oracle():
    for L in (1, 4, 32, 80):
        shp = api.shape(L)
        assert api.bytes_per_token(shp) == A.kv_bytes_per_token(L, 8, 128, 2)
        assert api.block_bytes(shp) == A.block_bytes(L, 8, 128, 2, 16)
    assert api.bytes_per_token(api.shape(80)) == 327_680
    assert api.block_bytes(api.shape(80)) == 5 * 2**20


def test_record_layout():
    size, offs = api.meta_layout()
    assert size == 64 == _abi.META_DTYPE.itemsize
    names = _abi.META_DTYPE.names
    assert offs == [_abi.META_DTYPE.fields[n][1] for n in names]


def test_workspace_sizing():
    shp = api.shape(80)
    sb = api.decode_split_blocks(shp, 1, 8192, 0, 80)
    assert sb in (16, 32, 64, 128, 256, 512, 1024)
    ws = api.decode_workspace_bytes(shp, 1, 8192, 8192, 0, 80, sb)
    # dominated by the mass partials: 4 B x 64 heads x 80 layers x 8192 blocks
    assert ws >= 4 * 64 * 80 * 8192
    assert ws < 4 * 64 * 80 * 8192 * 3
    assert api.decode_workspace_bytes(shp, 1, 8192, 8192, 0, 81, 0) == 0
    assert api.decode_split_blocks(shp, 1, 8192, 0, 80, 3) == 0
    assert api.decode_split_blocks(shp, 1, 8192, 0, 80, 64) == 64
    assert api.decode_split_blocks(shp, 1, 8192, 0, 80, 0, 3) == 0       # unknown format
    assert api.decode_workspace_bytes(shp, 1, 8192, 8192, 0, 80, 0, -1) == 0
    assert api.decode_split_blocks(shp, 1, 8192, 0, 80, 62, "kivi2") == 62
    assert api.decode_split_blocks(shp, 1, 8192, 0, 80, 63, "kivi2") == 0   # pairs need even splits
    assert api.decode_split_blocks(shp, 1, 8192, 0, 80, 63, "fp16") == 63


def test_split_policy():
    """The library's split choice keeps about 16 MiB of reads in flight on the
    chip and 56 KiB per compute unit, preferring the longest split."""
    def sb(batch, max_nb, layers, fmt):
        return api.decode_split_blocks(api.shape(layers), batch, max_nb, 0, layers, 0, fmt)
    assert sb(1, 8192, 80, "fp16") == 1024  # 128K context, fp16: 4 waves per CU suffice
    assert sb(1, 8192, 80, "e4m3") == 512   # E4M3: at most 512 blocks per split
    assert sb(1, 65536, 32, "fp16") == 1024
    assert sb(8, 512, 4, "fp16") == 128     # 1,024 waves x 16 KiB in flight
    assert sb(8, 512, 4, "e4m3") == 64      # E4M3 wants 2 waves per SIMD: 2,048 waves
    assert sb(1, 64, 1, "fp16") == 16       # too small to fill the chip: shortest split
    assert sb(1, 8192, 80, "kivi2") == 128  # issue-bound: at most 128 blocks per split
    assert sb(1, 256, 1, "kivi2") == 16     # 6 KiB per wave: 16 MiB in flight needs many waves
    assert api.score_workspace_bytes(1, 65536) >= 256 + 4 * 256
    assert api.score_workspace_bytes(0, 10) == 0


def _decode_args(**over):
    base = dict(shp=api.shape(2), q=0x1000, kv_pool=0x2000, pool_blocks=10, block_table=0x3000,
                max_blocks=4, seq_lens=0x4000, meta_offsets=0x5000, batch=2, total_blocks=8,
                layer_begin=0, layer_end=2, scale=0.088, out=0x6000, block_mass=0x7000,
                accumulate=0, split_blocks=0, workspace=0x10000, workspace_bytes=1)
    base.update(over)
    return base


def _decode(**over):
    a = _decode_args(**over)
    return api.decode_step(a["shp"], a["q"], a["kv_pool"], a["pool_blocks"], a["block_table"],
                           a["max_blocks"], a["seq_lens"], a["meta_offsets"], a["batch"],
                           a["total_blocks"], a["layer_begin"], a["layer_end"], a["scale"],
                           a["out"], a["block_mass"], a["accumulate"], a["split_blocks"],
                           a["workspace"], a["workspace_bytes"], stream=0)


@pytest.mark.parametrize("over,code", [
    (dict(q=0), KVS_E_NULL),
    (dict(kv_pool=0), KVS_E_NULL),
    (dict(block_mass=0), KVS_E_NULL),
    (dict(workspace=0), KVS_E_NULL),
    (dict(shp=api.Shape(2, 32, 8, 128, 16)), KVS_E_SHAPE),
    (dict(shp=api.Shape(2, 64, 8, 64, 16)), KVS_E_SHAPE),
    (dict(shp=api.Shape(0, 64, 8, 128, 16)), KVS_E_SHAPE),
    (dict(batch=0), KVS_E_RANGE),
    (dict(batch=65536), KVS_E_RANGE),
    (dict(max_blocks=1 << 27), KVS_E_RANGE),
    (dict(max_blocks=0), KVS_E_RANGE),
    (dict(pool_blocks=0), KVS_E_RANGE),
    (dict(layer_begin=1, layer_end=1), KVS_E_RANGE),
    (dict(layer_end=3), KVS_E_RANGE),
    (dict(scale=float("nan")), KVS_E_RANGE),
    (dict(accumulate=2), KVS_E_RANGE),
    (dict(split_blocks=2048), KVS_E_RANGE),
    (dict(total_blocks=-1), KVS_E_RANGE),
    (dict(q=0x1008), KVS_E_ALIGN),
    (dict(workspace=0x10010), KVS_E_ALIGN),
    (dict(), KVS_E_WORKSPACE),
])
def test_decode_rejects_before_launch(over, code):
    with pytest.raises(KvsError) as e:
        _decode(**over)
    assert e.value.code == code
    assert api.last_error()


def test_score_and_classify_validation():
    pol = api.policy(0.15)
    ok_ws = api.score_workspace_bytes(2, 4)
    args = (0x1000, 0x2000, 0x3000, 0x3800, 2, 4, 8)
    with pytest.raises(KvsError) as e:
        api.score_update(*args, 0, api.policy(0.0), 1, 0x10000, ok_ws, stream=0)
    assert e.value.code == KVS_E_POLICY
    with pytest.raises(KvsError) as e:
        api.score_update(*args, 0, api.policy(0.15, t_low=0.7, t_high=0.6), 1, 0x10000, ok_ws,
                         stream=0)
    assert e.value.code == KVS_E_POLICY
    with pytest.raises(KvsError) as e:
        api.score_update(*args, 0, api.policy(0.15, w_ema=-1.0), 1, 0x10000, ok_ws, stream=0)
    assert e.value.code == KVS_E_POLICY
    with pytest.raises(KvsError) as e:
        api.score_update(*args, 0, pol, 1, 0x10000, ok_ws - 4, stream=0)
    assert e.value.code == KVS_E_WORKSPACE
    with pytest.raises(KvsError) as e:
        api.score_update(*args, 2**64 - 1, pol, 1, 0x10000, ok_ws, stream=0)
    assert e.value.code == KVS_E_RANGE
    with pytest.raises(KvsError) as e:
        api.score_update(0, 0x2000, 0x3000, 0x3800, 2, 4, 8, 0, pol, 1, 0x10000, ok_ws, stream=0)
    assert e.value.code == KVS_E_NULL
    with pytest.raises(KvsError) as e:
        api.classify(0x1000, 0x3000, None, 0, 4, 8, pol, stream=0)
    assert e.value.code == KVS_E_RANGE
    with pytest.raises(KvsError) as e:
        api.meta_init(0x1000, 0x3000, 0x5000, 2, 4, 8, anchor_blocks=-1, stream=0)
    assert e.value.code == KVS_E_RANGE
    with pytest.raises(KvsError) as e:
        api.workspace_init(0x10000, 100, stream=0)
    assert e.value.code == KVS_E_WORKSPACE
    with pytest.raises(KvsError) as e:
        api.device_status(0, stream=0)
    assert e.value.code == KVS_E_NULL


def test_status_strings():
    for code in range(-7, 1):
        assert api.status_string(code) and api.status_string(code) != "unknown status"
    assert api.status_string(-99) == "unknown status"


def test_binding_requires_the_library(monkeypatch):
    monkeypatch.setattr(_abi, "_LIB", None)
    monkeypatch.setattr(_abi, "LIB_PATH", "/nonexistent/libkvs.so")
    with pytest.raises(ImportError):
        _abi.lib()


def test_append_validation():
    shp = api.shape(2)
    ws = api.append_workspace_bytes(3)
    assert ws >= 256 + 3 * 8
    base = dict(kv_elem_bytes=2, k_new=0x1000, v_new=0x2000, kv_pool=0x3000, pool_blocks=10,
                block_table=0x4000, max_blocks=4, seq_lens=0x5000, free_stack=0x6000,
                free_capacity=5, free_top=0x7000, meta=0x8000, meta_offsets=0x9000,
                seq_ids=0xA000, anchor_blocks=1, batch=3, total_blocks=12, workspace=0x10000,
                workspace_bytes=ws)

    def call(**over):
        a = dict(base, **over)
        api.append_kv(shp, a["kv_elem_bytes"], a["k_new"], a["v_new"], a["kv_pool"],
                      a["pool_blocks"], a["block_table"], a["max_blocks"], a["seq_lens"],
                      a["free_stack"], a["free_capacity"], a["free_top"], a["meta"],
                      a["meta_offsets"], a["seq_ids"], a["anchor_blocks"], a["batch"],
                      a["total_blocks"], a["workspace"], a["workspace_bytes"], stream=0)

    for over, code in [(dict(k_new=0), KVS_E_NULL), (dict(free_top=0), KVS_E_NULL),
                       (dict(kv_elem_bytes=4), KVS_E_RANGE), (dict(batch=0), KVS_E_RANGE),
                       (dict(free_capacity=-1), KVS_E_RANGE), (dict(anchor_blocks=-1), KVS_E_RANGE),
                       (dict(kv_pool=0x3008), KVS_E_ALIGN), (dict(workspace_bytes=ws - 1),
                                                             KVS_E_WORKSPACE)]:
        with pytest.raises(KvsError) as e:
            call(**over)
        assert e.value.code == code, over


def test_capacity_layout_host_side():
    import workload as W
    m = W.materialise(W.custom("cap", 1, [17, 40], seed=1, spare_blocks=5), "cpu",
                      extra_blocks=3)
    assert m.capacity == [2 + 3, 3 + 3]
    assert m.meta_offsets.tolist() == [0, 5, 11]
    assert m.total_blocks == 11 and m.max_blocks == 6
    assert m.block_table.shape == (2, 6)
    used = set(m.table_host[m.table_host >= 0].tolist())
    assert used.isdisjoint(set(m.free_stack.tolist()))
    assert len(used) + m.free_stack.size == m.pool_blocks


def _decode_kivi(kivi_pool=0x20000, kivi_blocks=4, quant_lens=0x30000, **over):
    a = _decode_args(**over)
    return api.decode_step_kivi(a["shp"], a["q"], a["kv_pool"], a["pool_blocks"], kivi_pool,
                                kivi_blocks, a["block_table"], a["max_blocks"], a["seq_lens"],
                                quant_lens, a["meta_offsets"], a["batch"], a["total_blocks"],
                                a["layer_begin"], a["layer_end"], a["scale"], a["out"],
                                a["block_mass"], a["accumulate"], a["split_blocks"],
                                a["workspace"], a["workspace_bytes"], stream=0)


@pytest.mark.parametrize("over,code", [
    (dict(kivi_pool=0), KVS_E_NULL),
    (dict(quant_lens=0), KVS_E_NULL),
    (dict(q=0), KVS_E_NULL),
    (dict(kivi_blocks=0), KVS_E_RANGE),
    (dict(kivi_blocks=1 << 31), KVS_E_RANGE),
    (dict(split_blocks=5), KVS_E_RANGE),            # 32-token pairs need even splits
    (dict(kivi_pool=0x20008), KVS_E_ALIGN),
    (dict(quant_lens=0x30002), KVS_E_ALIGN),
    (dict(), KVS_E_WORKSPACE),
])
def test_kivi_decode_rejects_before_launch(over, code):
    with pytest.raises(KvsError) as e:
        _decode_kivi(**over)
    assert e.value.code == code


def test_kivi_quantize_validation_and_sizes():
    shp = api.shape(80)
    assert api.kivi_block_bytes(shp) * 16 == api.block_bytes(shp) * 3   # 3 bits per element
    good = dict(kv_pool=0x1000, pool_blocks=8, kivi_pool=0x2000, kivi_blocks=8, pairs=0x3000,
                n_pairs=2, workspace=0x10000, workspace_bytes=256)
    cases = [(dict(kv_pool=0), KVS_E_NULL), (dict(pairs=0), KVS_E_NULL),
             (dict(n_pairs=-1), KVS_E_RANGE), (dict(kivi_blocks=0), KVS_E_RANGE),
             (dict(pool_blocks=1 << 31), KVS_E_RANGE), (dict(kivi_pool=0x2004), KVS_E_ALIGN),
             (dict(workspace=0x10004), KVS_E_ALIGN), (dict(workspace_bytes=255), KVS_E_WORKSPACE)]
    for over, code in cases:
        a = dict(good, **over)
        with pytest.raises(KvsError) as e:
            api.kivi_quantize(shp, a["kv_pool"], a["pool_blocks"], a["kivi_pool"],
                              a["kivi_blocks"], a["pairs"], a["n_pairs"], a["workspace"],
                              a["workspace_bytes"], stream=0)
        assert e.value.code == code, over
    # nothing to do: no launch, no error
    api.kivi_quantize(shp, 0x1000, 8, 0x2000, 8, 0x3000, 0, 0x10000, 256, stream=0)


def test_kivi_quant_len_rule_matches_the_oracle():
    """The library's window rule (kvs_kivi_quant_len, also applied on the device
    by kvs_kivi_advance) against the oracle's boundary, for several windows."""
    from oracle import kivi as KV
    for residual in (0, 1, 31, 32, 100, 128, 200):
        for n in list(range(0, 420)) + [131072, 1048576, 1048576 + 17]:
            assert api.kivi_quant_len(n, residual) == KV.quant_boundary(n, residual), (n, residual)
    assert api.kivi_quant_len(5000) == KV.quant_boundary(5000)     # the default window is 128
    with pytest.raises(ValueError):
        api.kivi_quant_len(-1)
    with pytest.raises(ValueError):
        api.kivi_quant_len(10, -3)


def test_binding_rejects_non_contiguous_tensors():
    import torch
    x = torch.zeros(4, 8)
    with pytest.raises(ValueError, match="contiguous"):
        api._p(x.t())
    assert api._p(x).value == x.data_ptr()



def _decode_paired(e4m3=False, pair_role=0x40000, **over):
    a = _decode_args(**over)
    fn = api.decode_step_e4m3_paired if e4m3 else api.decode_step_paired
    return fn(a["shp"], a["q"], a["kv_pool"], a["pool_blocks"], a["block_table"],
              a["max_blocks"], a["seq_lens"], pair_role, a["meta_offsets"], a["batch"],
              a["total_blocks"], a["layer_begin"], a["layer_end"], a["scale"], a["out"],
              a["block_mass"], a["accumulate"], a["split_blocks"], a["workspace"],
              a["workspace_bytes"], stream=0)


@pytest.mark.parametrize("e4m3", [False, True])
@pytest.mark.parametrize("over,code", [
    (dict(pair_role=0), KVS_E_NULL),
    (dict(q=0), KVS_E_NULL),
    (dict(pair_role=0x40002), KVS_E_ALIGN),
    (dict(split_blocks=1024), KVS_E_RANGE),       # a paired split holds at most 512 blocks
    (dict(batch=0), KVS_E_RANGE),
    (dict(), KVS_E_WORKSPACE),
])
def test_paired_decode_rejects_before_launch(e4m3, over, code):
    with pytest.raises(KvsError) as e:
        _decode_paired(e4m3=e4m3, **over)
    assert e.value.code == code
    assert api.last_error()


def test_layer_count_is_bounded_before_any_size_is_formed():
    # 65,536 layers would take the workspace sizes towards 64-bit overflow
    big = api.Shape(65536, 64, 8, 128, 16)
    assert api.decode_workspace_bytes(big, 1, 16, 16, 0, 65536, 0, "fp16") == 0
    with pytest.raises(KvsError) as e:
        _decode(shp=big, layer_end=1)
    assert e.value.code == KVS_E_SHAPE
    ok = api.Shape(65535, 64, 8, 128, 16)
    assert api.decode_workspace_bytes(ok, 1, 16, 16, 0, 1, 0, "fp16") > 0


def _decode_noalloc(status=0x8000, **over):
    a = _decode_args(**over)
    return api.decode_step_noalloc(a["shp"], a["q"], a["kv_pool"], a["pool_blocks"],
                                   a["block_table"], a["max_blocks"], a["seq_lens"],
                                   a["meta_offsets"], a["batch"], a["total_blocks"],
                                   a["layer_begin"], a["layer_end"], a["scale"], a["out"],
                                   a["block_mass"], a["accumulate"], a["split_blocks"], status,
                                   stream=0)


@pytest.mark.parametrize("over,code", [
    (dict(status=0), KVS_E_NULL),
    (dict(status=0x8002), KVS_E_ALIGN),
    (dict(q=0), KVS_E_NULL),
    (dict(block_mass=0), KVS_E_NULL),
    (dict(batch=0), KVS_E_RANGE),
    (dict(layer_end=3), KVS_E_RANGE),
    (dict(split_blocks=2048), KVS_E_RANGE),
    (dict(q=0x1008), KVS_E_ALIGN),
    # 128K tokens x 80 layers in one call needs ~165 MiB of split partials
    (dict(shp=api.shape(80), layer_end=80, max_blocks=8192, total_blocks=8192, batch=1),
     KVS_E_WORKSPACE),
])
def test_noalloc_decode_rejects_before_launch(over, code):
    """Every host check of kvs_decode_step_noalloc returns before the library
    looks up its scratch or launches anything (no GPU here)."""
    with pytest.raises(KvsError) as e:
        _decode_noalloc(**over)
    assert e.value.code == code
    if code == KVS_E_WORKSPACE:
        assert "layer range" in e.value.message


def test_noalloc_scratch_holds_a_layer_range_of_the_128k_step():
    """The 32 MiB scratch takes the 128K-token step in ranges of 8 layers."""
    shp = api.shape(80)
    assert _abi.KVS_NOALLOC_SCRATCH_BYTES == 32 << 20
    assert api.decode_workspace_bytes(shp, 1, 8192, 8192, 0, 8, 0, "fp16") <= 32 << 20
    assert api.decode_workspace_bytes(shp, 1, 8192, 8192, 0, 80, 0, "fp16") > 32 << 20


def test_stream_probe_rejects_small_buffers_before_the_library():
    """The binding checks tensor sizes against the probe's contract (read mode
    writes grid x 256 words; copy mode writes nbytes) and raises before any
    device call."""
    import torch
    src = torch.zeros(1024, dtype=torch.int32)
    with pytest.raises(ValueError):
        api.stream_probe(src, torch.zeros(4, dtype=torch.int32), 4096, 0)          # 2048 x 256 words
    with pytest.raises(ValueError):
        api.stream_probe(src, torch.zeros(255, dtype=torch.int32), 4096, 0, grid=1)
    with pytest.raises(ValueError):
        api.stream_probe(src, torch.zeros(1023, dtype=torch.int32), 4096, 1)
    with pytest.raises(ValueError):
        api.stream_probe(src, torch.zeros(1024, dtype=torch.int32), 8192, 1)     # src too small


def test_last_error_is_set_by_a_failure_and_cleared_by_a_success():
    """kvs_last_error: the failing call's message, then "" after a call that
    returns KVS_OK (no device work: the decode-event hook only stores handles)."""
    with pytest.raises(Exception):
        api.set_decode_events(1, None)
    assert "neither" in api.last_error()
    api.set_decode_events(None, None)
    assert api.last_error() == ""
