"""GPU parity of the KIVI 2-bit KV path (kvs_kivi_quantize, kvs_decode_step_kivi)
against the oracle's quantisation, packed format and decode (oracle/kivi.py)."""
import math

import numpy as np
import pytest
import torch

import workload as W
from oracle import kivi as KV
from oracle import scoring as OS
from paged_gqa_kv_amd import api
from paged_gqa_kv_amd.session import DecodeSession

from . import parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda"
SCALE = 1.0 / math.sqrt(128.0)


def _case(msg):
    print(f"\n[case] {msg}", flush=True)


def _kivi_session(lens, layers=2, split_blocks=0, seed=21, shared=0):
    wl = W.as_kivi2(W.custom("kivi", layers, lens, seed=seed, spare_blocks=7,
                             shared_prefix_tokens=shared))
    m = W.materialise(wl, DEV)
    sess = DecodeSession(m, split_blocks=split_blocks)
    torch.cuda.synchronize()
    assert [api.kivi_quant_len(n) for n in m.lens] == [KV.quant_boundary(n) for n in m.lens]
    return m, sess


def _check_quantised_bytes(m, sess, layers_to_check=None):
    pool = m.pool.cpu().numpy()
    kivi = sess.kivi_pool.cpu().numpy().reshape(sess.kivi_blocks, m.num_layers, 2, 8, KV.TILE_BYTES)
    ktab = sess.kivi_table_host
    layers = range(m.num_layers) if layers_to_check is None else layers_to_check
    checked = 0
    for s in range(m.batch):
        for p in range(int(sess.quant_lens_host[s]) // 32):
            e, o = m.table_host[s, 2 * p], m.table_host[s, 2 * p + 1]
            de, do = ktab[s, 2 * p], ktab[s, 2 * p + 1]
            for layer in layers:
                for g in range(8):
                    K32 = np.concatenate([pool[e, layer, 0, g], pool[o, layer, 0, g]])
                    V32 = np.concatenate([pool[e, layer, 1, g], pool[o, layer, 1, g]])
                    ke, ko, ve, vo = KV.pack_pair(K32, V32)
                    assert kivi[de, layer, 0, g].tobytes() == ke, (s, p, layer, g, "K even")
                    assert kivi[do, layer, 0, g].tobytes() == ko, (s, p, layer, g, "K odd")
                    assert kivi[de, layer, 1, g].tobytes() == ve, (s, p, layer, g, "V even")
                    assert kivi[do, layer, 1, g].tobytes() == vo, (s, p, layer, g, "V odd")
                    checked += 1
    return checked


def test_quantiser_writes_the_oracles_bytes():
    _case("kvs_kivi_quantize vs the oracle's packed tiles, 2 layers, lengths 200/33/500/1000")
    m, sess = _kivi_session([200, 33, 500, 1000])
    n = _check_quantised_bytes(m, sess)
    assert n == 2 * 8 * sum(KV.quant_boundary(x) // 32 for x in m.lens)
    assert sess.status() == 0


def test_quantiser_edge_values():
    _case("quantiser on degenerate and outlier groups: constant channels, one huge channel")
    wl = W.as_kivi2(W.custom("kedge", 1, [288], seed=5, spare_blocks=3))
    m = W.materialise(wl, DEV)
    # constant key channel 3, huge key channel 77, constant value group of token 10
    pids = torch.as_tensor(m.table_host[0, :18].astype(np.int64), device=DEV)
    blk = m.pool[pids]                                    # [18][L][2][8][16][128]
    blk[:, :, 0, :, :, 3] = 0.75
    blk[:, :, 0, :, :, 77] *= 500.0
    blk[0, :, 1, :, 10, 32:64] = -1.5
    m.pool[pids] = blk
    sess = DecodeSession(m)
    torch.cuda.synchronize()
    assert _check_quantised_bytes(m, sess) > 0


@pytest.mark.parametrize("split_blocks", [0, 4, 16, 64])
def test_kivi_decode_parity(split_blocks):
    _case(f"KIVI decode vs oracle, 2 layers, ragged lengths, split_blocks={split_blocks}")
    m, sess = _kivi_session([1, 17, 159, 160, 161, 200, 333, 1000, 2049], split_blocks=split_blocks)
    pool = m.pool.cpu().numpy()
    for step in range(2):
        q = W.make_query(m, step)
        sess.decode(q)
        torch.cuda.synchronize()
        out_ref, mass_ref = KV.decode_step(q.cpu().numpy(), pool, m.table_host, m.lens, SCALE)
        w_out = P.check_out(sess.out, out_ref, range(m.num_layers))
        w_mass = P.check_mass(sess.mass, mass_ref, m.meta_offsets.cpu().numpy())
        print(f"  step {step}: worst output {w_out:.2e}, worst mass {w_mass:.2e}", flush=True)
    assert sess.status() == 0


def test_kivi_decode_shared_prefix_and_scoring():
    _case("KIVI decode + scoring, shared 256-token prefix quantised once, 3 layers, 4 steps")
    m, sess = _kivi_session([300, 640, 256, 1200], layers=3, shared=256, seed=4)
    shared_pairs = sum(KV.quant_boundary(n) // 32 for n in m.lens)
    assert int(sess.kivi_pairs.shape[0]) < shared_pairs          # shared pairs quantised once
    _check_quantised_bytes(m, sess, layers_to_check=[1])
    pool = m.pool.cpu().numpy()
    pol = OS.Policy(alpha=0.15)
    gpol = api.policy(0.15)
    state = OS.init_state(m.blocks, m.seq_ids.cpu().numpy())
    for step in range(4):
        q = W.make_query(m, step)
        sess.step(q, step, gpol)
        torch.cuda.synchronize()
        out_ref, mass_ref = KV.decode_step(q.cpu().numpy(), pool, m.table_host, m.lens, SCALE)
        P.check_out(sess.out, out_ref, range(m.num_layers))
        P.check_mass(sess.mass, mass_ref, m.meta_offsets.cpu().numpy())
        state, stale = OS.score_update(state, mass_ref, step, pol)
        assert not stale.any()
        P.check_records(sess.records(), state, pol)
    assert sess.status() == 0


def test_kivi_bad_quant_len_skips_the_sequence():
    _case("quant_lens not a multiple of 32 / beyond the length: status bit, zero output")
    m, sess = _kivi_session([500, 400])
    q = W.make_query(m, 0)
    good = sess.quant_lens.clone()
    for bad in (good[0] - 16, torch.tensor(512, dtype=torch.int32, device=DEV)):
        sess.quant_lens[0] = bad
        sess.decode(q)
        torch.cuda.synchronize()
        assert sess.status() & api._abi.KVS_DEV_BAD_SEQ_LEN
        assert torch.count_nonzero(sess.out[0]) == 0
        offs = m.meta_offsets.cpu().numpy()
        assert torch.count_nonzero(sess.mass[offs[0]:offs[1]]) == 0
        out_ref, mass_ref = KV.decode_step(q[1:].cpu().numpy(), m.pool.cpu().numpy(),
                                           m.table_host[1:], m.lens[1:], SCALE)
        P.check_out(sess.out[1:], out_ref, range(m.num_layers))
    sess.quant_lens.copy_(good)
    sess.decode(q)
    torch.cuda.synchronize()
    assert sess.status() == 0


def test_kivi_append_moves_the_boundary():
    """70 steps of append -> advance -> decode -> score on KIVI caches.  The
    oracle keeps every token's fp16 K/V and applies the window rule itself, so
    it is independent of which fp16 blocks the GPU freed and reused."""
    _case("KIVI append + boundary advance + decode + score, 70 steps, 2 layers")
    lens0 = [150, 159, 190, 300, 47]
    wl = W.as_kivi2(W.custom("kapp", 2, lens0, seed=17, spare_blocks=40))
    m = W.materialise(wl, DEV, extra_blocks=6)
    sess = DecodeSession(m, kivi_spare_blocks=30)
    L, B = m.num_layers, m.batch
    pool = m.pool.cpu().numpy()
    hist_k, hist_v = [], []
    for s in range(B):
        pids = m.table_host[s, :m.blocks[s]]
        blk = pool[pids]                                          # [nb][L][2][8][16][128]
        kv = blk.transpose(1, 2, 3, 0, 4, 5).reshape(L, 2, 8, -1, 128)[:, :, :, :m.lens[s]]
        hist_k.append(kv[:, 0].copy())
        hist_v.append(kv[:, 1].copy())
    lens = list(m.lens)
    pol = OS.Policy(alpha=0.15)
    gpol = api.policy(0.15)
    offsets = m.meta_offsets.cpu().numpy()
    state = OS.init_state(m.blocks, m.seq_ids.cpu().numpy())
    top = int(m.free_stack.size)
    for step in range(70):
        k, v = W.new_token_kv(m, step)
        top_before = int(sess.free_top.item()) if hasattr(sess, "free_top") else top
        sess.append(k, v)
        kh, vh = k.cpu().numpy(), v.cpu().numpy()
        opened = advanced = 0
        for s in range(B):
            hist_k[s] = np.concatenate([hist_k[s], kh[s][:, :, None]], axis=2)
            hist_v[s] = np.concatenate([hist_v[s], vh[s][:, :, None]], axis=2)
            opened += lens[s] % 16 == 0
            advanced += KV.quant_boundary(lens[s] + 1) > KV.quant_boundary(lens[s])
            lens[s] += 1
        q = W.make_query(m, step)
        sess.decode(q)
        sess.score(step, gpol)
        torch.cuda.synchronize()
        assert m.seq_lens.cpu().tolist() == lens
        assert sess.quant_lens.cpu().tolist() == [KV.quant_boundary(n) for n in lens]
        assert int(sess.free_top.item()) == top_before - opened + 2 * advanced
        # decode against the oracle on the full history
        qh = q.cpu().numpy()
        out_ref = np.full(qh.shape, np.nan)
        mass_ref = []
        for s in range(B):
            mass = np.zeros(-(-lens[s] // 16))
            for layer in range(L):
                for g in range(8):
                    Kh, Vh = KV.kivi_kv(hist_k[s][layer, g], hist_v[s][layer, g], lens[s])
                    for h in range(8 * g, 8 * g + 8):
                        out_ref[s, layer, h], p = KV.OA.attend_head(qh[s, layer, h], Kh, Vh, SCALE)
                        mass += KV.OA.block_sums(p, lens[s])
            mass_ref.append(mass)
        P.check_out(sess.out, out_ref, range(L))
        P.check_mass(sess.mass, mass_ref, offsets)
        blocks = [-(-n // 16) for n in lens]
        state = OS.grow(state, blocks)
        state, stale = OS.score_update(state, mass_ref, step, pol)
        assert not stale.any()
        rows = np.concatenate([offsets[s] + np.arange(nb) for s, nb in enumerate(blocks)])
        P.check_records(sess.records()[rows], state, pol)
    # every pair quantised along the way holds the oracle's bytes
    kivi = sess.kivi_pool.cpu().numpy().reshape(sess.kivi_blocks, L, 2, 8, KV.TILE_BYTES)
    tab = sess.kivi_table.cpu().numpy()
    for s in range(B):
        for p in range(KV.quant_boundary(lens[s]) // 32):
            de, do = tab[s, 2 * p], tab[s, 2 * p + 1]
            for layer in range(L):
                for g in range(8):
                    ke, ko, ve, vo = KV.pack_pair(hist_k[s][layer, g, 32 * p:32 * p + 32],
                                                  hist_v[s][layer, g, 32 * p:32 * p + 32])
                    assert kivi[de, layer, 0, g].tobytes() == ke and kivi[do, layer, 0, g].tobytes() == ko
                    assert kivi[de, layer, 1, g].tobytes() == ve and kivi[do, layer, 1, g].tobytes() == vo
    assert sess.status() == 0


def test_kivi_advance_without_free_quantised_blocks():
    _case("kvs_kivi_advance with one free quantised block: boundary kept, status bit")
    wl = W.as_kivi2(W.custom("kex", 1, [159, 159], seed=2, spare_blocks=8))
    m = W.materialise(wl, DEV, extra_blocks=2)
    sess = DecodeSession(m, kivi_spare_blocks=3)      # 2 initial-free ids after 0 pairs, +1
    assert int(sess.kivi_free_host.size) == 3
    k, v = W.new_token_kv(m, 0)
    sess.append(k, v)                                  # 160 tokens: both sequences want a pair
    torch.cuda.synchronize()
    assert sess.quant_lens.cpu().tolist() == [32, 0]   # the first takes two ids, the second finds one
    assert int(sess.kivi_free_top.item()) == 1
    assert sess.status() & api._abi.KVS_DEV_POOL_EXHAUSTED
    q = W.make_query(m, 0)
    sess.decode(q)
    torch.cuda.synchronize()
    lens = m.seq_lens.cpu().tolist()
    assert lens == [160, 160]


def test_kivi_advance_batch_larger_than_one_work_group():
    """1,300 sequences at 159 tokens all cross the window on the same append:
    allocation scans two chunks and the commit kernel walks 1,300 jobs."""
    _case("kvs_kivi_advance with 1300 simultaneous boundary moves, 1 layer")
    wl = W.as_kivi2(W.custom("kwide", 1, [159] * 1300, seed=9, spare_blocks=2700))
    m = W.materialise(wl, DEV, extra_blocks=2)
    sess = DecodeSession(m, kivi_spare_blocks=2 * 1300)
    free0 = sess.kivi_free_host.copy()
    k, v = W.new_token_kv(m, 0)
    sess.append(k, v)
    torch.cuda.synchronize()
    assert sess.status() == 0
    assert sess.quant_lens.cpu().tolist() == [32] * 1300
    assert int(sess.kivi_free_top.item()) == 0
    tab = sess.kivi_table.cpu().numpy()
    # batch order from the top of the stack: sequence s takes free0[-1 - 2s], free0[-2 - 2s]
    for s in (0, 1, 1023, 1024, 1299):
        assert tab[s, 0] == free0[free0.size - 1 - 2 * s] and tab[s, 1] == free0[free0.size - 2 - 2 * s]
    # the freed fp16 blocks went onto the append stack, pair by pair in batch order
    top = int(sess.free_top.item())
    stack = sess.free_stack.cpu().numpy()
    pushed = stack[top - 2 * 1300:top].reshape(1300, 2)
    assert np.array_equal(pushed, m.table_host[:, :2].astype(np.int32))
    kivi = sess.kivi_pool.cpu().numpy().reshape(sess.kivi_blocks, 1, 2, 8, KV.TILE_BYTES)
    pool = m.pool.cpu().numpy()
    for s in (0, 1024, 1299):
        e, o = m.table_host[s, 0], m.table_host[s, 1]
        for g in (0, 7):
            K32 = np.concatenate([pool[e, 0, 0, g], pool[o, 0, 0, g]])
            V32 = np.concatenate([pool[e, 0, 1, g], pool[o, 0, 1, g]])
            ke, ko, ve, vo = KV.pack_pair(K32, V32)
            assert kivi[tab[s, 0], 0, 0, g].tobytes() == ke and kivi[tab[s, 1], 0, 1, g].tobytes() == vo


def test_mixed_precision_by_layer():
    """fp16 for the first layer, KIVI for the rest (the per-layer escape hatch of
    Fitting a Million Tokens, Sec. 02): two calls over layer ranges, the second
    accumulating the block mass."""
    _case("layer 0 fp16 + layers 1..2 KIVI, block mass accumulated across the two calls")
    from oracle import attention as OA
    m, sess = _kivi_session([600, 200, 1300], layers=3, seed=31)
    import dataclasses
    m16 = type(m)(**{**m.__dict__, "workload": dataclasses.replace(m.workload, kv_format="fp16")})
    fp16 = DecodeSession(m16, layer_begin=0, layer_end=1)
    q = W.make_query(m, 0)
    fp16.decode(q)                                            # layer 0, fp16 pool
    sess.mass.copy_(fp16.mass)
    sess.decode(q, accumulate=1, layer_begin=1, layer_end=3)  # layers 1-2, KIVI cache
    torch.cuda.synchronize()
    pool = m.pool.cpu().numpy()
    qh = q.cpu().numpy()
    out0, mass0 = OA.decode_step(qh, pool, m.table_host, m.lens, SCALE, 0, 1)
    out12, mass12 = KV.decode_step(qh, pool, m.table_host, m.lens, SCALE, 1, 3)
    P.check_out(fp16.out, out0, [0])
    P.check_out(sess.out, out12, [1, 2])
    P.check_mass(sess.mass, [a + b for a, b in zip(mass0, mass12)], m.meta_offsets.cpu().numpy())
    assert sess.status() == 0 and fp16.status() == 0


@pytest.mark.parametrize("bad_top", [-7, 1 << 20])
def test_kivi_advance_clamps_an_out_of_range_fp16_free_top(bad_top):
    """kivi_advance_commit clamps a top outside [0, capacity] (here -7 and far
    above the capacity) into the stack before pushing, and reports
    KVS_DEV_BAD_OFFSETS: the pushes land inside the stack."""
    _case(f"kvs_kivi_advance with fp16_free_top = {bad_top}")
    wl = W.as_kivi2(W.custom("kclamp", 1, [159, 100], seed=3, spare_blocks=8))
    m = W.materialise(wl, DEV, extra_blocks=2)
    sess = DecodeSession(m, kivi_spare_blocks=4)
    assert sess.quant_lens.cpu().tolist() == [0, 0]
    m.seq_lens[0] = 160      # token 159 sits in slot 15 of its block: the window is full
    cap = 6
    fp16_free = torch.full((cap,), -1, dtype=torch.int32, device=DEV)
    fp16_top = torch.tensor([bad_top], dtype=torch.int32, device=DEV)
    kivi_free = torch.from_numpy(sess.kivi_free_host.astype(np.int32)).to(DEV)
    kivi_top = torch.tensor([int(sess.kivi_free_host.size)], dtype=torch.int32, device=DEV)
    ws = torch.empty(api.kivi_advance_workspace_bytes(m.batch), dtype=torch.uint8, device=DEV)
    api.workspace_init(ws)
    api.kivi_advance(sess.shape, m.pool, m.pool_blocks, sess.kivi_pool, sess.kivi_blocks,
                     sess.kivi_table, m.max_blocks, m.seq_lens, sess.quant_lens, m.batch,
                     api.KIVI_RESIDUAL_TOKENS, kivi_free, int(kivi_free.numel()), kivi_top,
                     fp16_free, cap, fp16_top, ws)
    torch.cuda.synchronize()
    assert api.device_status(ws) & api._abi.KVS_DEV_BAD_OFFSETS
    assert sess.quant_lens.cpu().tolist() == [32, 0]
    start = 0 if bad_top < 0 else cap
    pushed = fp16_free.cpu().tolist()
    if start + 2 <= cap:
        assert pushed[:2] == m.table_host[0, :2].tolist() and int(fp16_top.item()) == 2
    else:   # clamped to a full stack: nothing fits, the ids are not pushed
        assert pushed == [-1] * cap and int(fp16_top.item()) == cap
