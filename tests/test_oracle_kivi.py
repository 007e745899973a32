"""Pins for the oracle's KIVI 2-bit KV (Fitting a Million Tokens, Sec. 02)."""
import math

import numpy as np
import pytest

import workload as W
from oracle import attention as OA
from oracle import kivi as KV


def _f16(x):
    return np.asarray(x, dtype=np.float16)


def test_exact_grid_round_trips():
    # every group spans exactly {z, z+s, z+2s, z+3s} with s a power of two:
    # span / 3 = s is exact, so the codes are the grid indices and read back exactly
    rng = np.random.default_rng(0)
    idx = rng.integers(0, 4, size=(5, 32))
    idx[:, 0], idx[:, 1] = 0, 3                             # both ends present
    z = _f16([-1.5, 0.0, 2.0, -0.25, 7.0])[:, None]
    s = _f16([0.5, 0.125, 1.0, 0.0625, 2.0])[:, None]
    x = _f16(z.astype(np.float64) + idx * s.astype(np.float64))
    codes, sc, ze = KV.quantize_groups(x, axis=1)
    assert np.array_equal(codes, idx)
    assert np.array_equal(sc, s[:, 0]) and np.array_equal(ze, z[:, 0])
    assert np.array_equal(KV.dequantize(codes, sc, ze, axis=1), x.astype(np.float64))


def test_read_back_within_half_a_step():
    rng = np.random.default_rng(1)
    x = _f16(rng.standard_normal((2000, 32)) * rng.uniform(0.01, 50, size=(2000, 1)))
    codes, s, z = KV.quantize_groups(x, axis=1)
    xh = KV.dequantize(codes, s, z, axis=1)
    err = np.abs(xh - x.astype(np.float64))
    step = s.astype(np.float64)[:, None]
    # half a step, plus the fp16 rounding of the step (the top code may land a
    # relative 2^-11 of the span short of the maximum)
    assert np.all(err <= step * (0.5 + 2.0 ** -9))
    assert codes.max() == 3 and codes.min() == 0
    # min and max of each group are reproduced to within that rounding
    assert np.all(np.abs(xh.min(axis=1) - x.astype(np.float64).min(axis=1)) == 0)


def test_equal_elements_give_scale_zero_and_exact_read_back():
    # the degenerate group the section warns about: min equals max, the scale
    # collapses and the round trip is exact
    x = _f16(np.full((3, 32), [[1.25], [-3.0], [0.0]]))
    codes, s, z = KV.quantize_groups(x, axis=1)
    assert np.all(s == 0) and np.all(codes == 0)
    assert np.array_equal(KV.dequantize(codes, s, z, axis=1), x.astype(np.float64))


def test_brute_force_groups_scales_codes():
    """Pure-Python loops over a tiny tensor: keys grouped per channel over 32
    tokens, values per token over 32 channels."""
    rng = np.random.default_rng(2)
    n, d = 64, 128
    K = _f16(rng.standard_normal((n, d)))
    V = _f16(rng.standard_normal((n, d)))
    kc, ks, kz = KV.quantize_keys(K)
    vc, vs, vz = KV.quantize_values(V)
    assert ks.shape == (n // 32, d) and vs.shape == (n, d // 32)

    def one(vals):
        vals = [float(v) for v in vals]
        lo, hi = min(vals), max(vals)
        sc = float(np.float16(np.float32(np.float32(hi - lo) / np.float32(3))))
        cs = []
        for v in vals:
            if sc == 0.0:
                cs.append(0)
                continue
            t = float(np.float32(np.float32(v - lo) / np.float32(sc)))
            r = math.floor(t + 0.5) if t - math.floor(t) != 0.5 else (
                math.floor(t) if math.floor(t) % 2 == 0 else math.floor(t) + 1)
            cs.append(min(3, max(0, r)))
        return lo, sc, cs

    for grp in range(n // 32):
        for ch in (0, 5, 31, 32, 77, 127):
            lo, sc, cs = one(K[32 * grp:32 * grp + 32, ch])
            assert float(kz[grp, ch]) == lo and float(ks[grp, ch]) == sc
            assert list(kc[32 * grp:32 * grp + 32, ch]) == cs
    for tok in (0, 1, 17, 40, 63):
        for g in range(4):
            lo, sc, cs = one(V[tok, 32 * g:32 * g + 32])
            assert float(vz[tok, g]) == lo and float(vs[tok, g]) == sc
            assert list(vc[tok, 32 * g:32 * g + 32]) == cs


def test_outlier_channel_stays_in_its_own_key_groups():
    # the asymmetry argument of the section: a persistent outlier channel,
    # quantised per channel, does not widen the other channels' steps
    rng = np.random.default_rng(3)
    K = rng.standard_normal((96, 128))
    K[:, 9] = 300.0 + 20.0 * K[:, 9]             # persistent large channel
    K = _f16(K)
    Kh = KV.dequantize_keys(*KV.quantize_keys(K))
    err = np.abs(Kh - K.astype(np.float64))
    normal = np.delete(np.arange(128), 9)
    assert err[:, normal].max() < 1.5           # half the step of a unit-variance channel
    assert err[:, 9].max() > 5.0                # the outlier's own step is wide
    kc, _, _ = KV.quantize_keys(K)
    assert all(len(np.unique(kc[:, ch])) == 4 for ch in normal)
    # grouping keys per token instead lets the outlier set the step of its
    # 32-channel group: the other 31 channels collapse onto the lowest level
    vc, _, _ = KV.quantize_values(K)
    same_group = [ch for ch in range(32) if ch != 9]
    assert vc[:, same_group].max() == 0


def test_boundary_rule():
    cases = {0: 0, 1: 0, 100: 0, 128: 0, 159: 0, 160: 32, 191: 32, 192: 64, 1000: 864,
             131072: 130944}
    for n, nq in cases.items():
        assert KV.quant_boundary(n) == nq, n
        assert nq % 32 == 0
        if n >= 160:
            assert 128 <= n - nq < 160


def test_effective_bits_and_compression():
    # the section's arithmetic: an fp16 scale and zero per 32-element group is
    # one extra bit per element, so 2-bit codes are ~3 bits and 16 / 3 ~ 5.3x
    tile_fp16 = 16 * 128 * 2
    assert KV.TILE_BYTES * 8 / (16 * 128) == 3.0
    assert round(tile_fp16 / KV.TILE_BYTES, 1) == 5.3
    # the residual window of ~128 tokens costs about 40 MB on the 70B shape
    per_token = 2 * 80 * 8 * 128 * 2
    assert 40e6 < 128 * per_token < 43e6


def test_packed_format_hand_placed_bits():
    # key tile: code 3 at token 5, channel 37 -> j = (37 % 32) // 8 = 0, entry 5,
    # set i = 1, m = 5 -> word 0, bit 4 * 5 + 2 = 22 -> byte 8 * 5 + 2, bits 6..7
    codes = np.zeros((16, 128), np.uint8)
    codes[5, 37] = 3
    raw = KV.pack_k_tile(codes, np.zeros(128, np.float16), np.zeros(128, np.float16), False)
    b = np.frombuffer(raw[:512], np.uint8)
    assert b[42] == 0xC0 and b.sum() == 0xC0
    # value tile: code 2 at token 9, channel 70 -> j = 9 // 4 = 2, r = 1, tile
    # k = 70 // 16 = 4, c = 6 -> entry 38, set 2, m = 1 -> word 1, bit 4 -> byte
    # 8 * 38 + 4, value 2 << 4
    codes = np.zeros((16, 128), np.uint8)
    codes[9, 70] = 2
    raw = KV.pack_v_tile(codes, np.zeros((16, 4), np.float16), np.zeros((16, 4), np.float16))
    b = np.frombuffer(raw[:512], np.uint8)
    assert b[8 * 38 + 4] == 0x20 and b.sum() == 0x20
    # parameters: key channel 70 of an odd block: scale at 512 + 2 * 6, zero at
    # 640 + 2 * 6; value token 9, group 2: scale at 512 + 2 * 41, zero at 640 + 82
    s = np.zeros(128, np.float16)
    z = np.zeros(128, np.float16)
    s[70], z[70] = 1.5, -0.25
    raw = KV.pack_k_tile(np.zeros((16, 128), np.uint8), s, z, True)
    meta = np.frombuffer(raw[512:], "<f2")
    assert meta[6] == 1.5 and meta[64 + 6] == -0.25 and np.count_nonzero(meta) == 2
    vs = np.zeros((16, 4), np.float16)
    vz = np.zeros((16, 4), np.float16)
    vs[9, 2], vz[9, 2] = -2.0, 3.0
    raw = KV.pack_v_tile(np.zeros((16, 128), np.uint8), vs, vz)
    meta = np.frombuffer(raw[512:], "<f2")
    assert meta[41] == -2.0 and meta[64 + 41] == 3.0 and np.count_nonzero(meta) == 2


def test_pack_unpack_round_trip_and_layout_is_a_bijection():
    rng = np.random.default_rng(4)
    for layout in (KV.k_entry_layout, KV.v_entry_layout):
        t, d = layout()
        pairs = set(zip(t.ravel().tolist(), d.ravel().tolist()))
        assert len(pairs) == 16 * 128
    codes = rng.integers(0, 4, (16, 128)).astype(np.uint8)
    s = _f16(rng.standard_normal(128))
    z = _f16(rng.standard_normal(128))
    for odd in (False, True):
        c2, s2, z2 = KV.unpack_k_tile(KV.pack_k_tile(codes, s, z, odd))
        half = slice(64, 128) if odd else slice(0, 64)
        assert np.array_equal(c2, codes) and np.array_equal(s2, s[half]) and np.array_equal(z2, z[half])
    vs = _f16(rng.standard_normal((16, 4)))
    vz = _f16(rng.standard_normal((16, 4)))
    c2, s2, z2 = KV.unpack_v_tile(KV.pack_v_tile(codes, vs, vz))
    assert np.array_equal(c2, codes) and np.array_equal(s2, vs) and np.array_equal(z2, vz)


def _grid_pool(m, rng):
    """Replace live K/V with values every 32-token key group and every 32-channel
    value group of which lies on an exact 4-level grid (lossless quantisation)."""
    pool = m.pool.numpy().copy()
    for s in range(m.batch):
        n = m.lens[s]
        nq = KV.quant_boundary(n)
        for b in range(nq // 16):
            pid = m.table_host[s, b]
            grp = b // 2
            for layer in range(m.num_layers):
                # keys: per channel the same (z, s) across the 32-token group
                zk = (np.arange(128) % 7 - 3) * 0.25 + 0.0625 * grp
                k = zk + rng.integers(0, 4, (16, 8, 128)) * 0.5
                k[0, :, :] = zk if b % 2 == 0 else k[0]
                k[1, :, :] = zk + 1.5 if b % 2 == 0 else k[1]
                pool[pid, layer, 0] = k.transpose(1, 0, 2)
                # values: per token, each 32-channel group on its own grid
                zv = np.repeat(rng.integers(-4, 4, (8, 16, 4)) * 0.5, 32, axis=2)
                v = zv + rng.integers(0, 4, (8, 16, 128)) * 0.25
                v[..., ::32] = zv[..., ::32]
                v[..., 1::32] = zv[..., 1::32] + 0.75
                pool[pid, layer, 1] = v
    return pool


def test_decode_over_lossless_cache_equals_fp16_decode():
    rng = np.random.default_rng(5)
    m = W.materialise(W.custom("kgrid", 2, [200, 96, 330], seed=6), "cpu")
    pool = _grid_pool(m, rng)
    q = rng.standard_normal((m.batch, 2, 64, 128)).astype(np.float16)
    scale = 1.0 / math.sqrt(128.0)
    o1, m1 = KV.decode_step(q, pool, m.table_host, m.lens, scale)
    o2, m2 = OA.decode_step(q, pool, m.table_host, m.lens, scale)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    for a, b in zip(m1, m2):
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=0)
    # and the quantised part really was quantised: random (off-grid) data differs
    o3, _ = KV.decode_step(q, m.pool.numpy(), m.table_host, m.lens, scale)
    o4, _ = OA.decode_step(q, m.pool.numpy(), m.table_host, m.lens, scale)
    assert np.abs(o3[0] - o4[0]).max() > 1e-3           # sequence 0 has 200 tokens: 64 quantised
    assert np.array_equal(o3[1], o4[1])                   # 96 tokens: all in the fp16 window


def test_short_sequences_are_untouched():
    rng = np.random.default_rng(7)
    m = W.materialise(W.custom("kshort", 1, [1, 17, 159], seed=8), "cpu")
    q = rng.standard_normal((m.batch, 1, 64, 128)).astype(np.float16)
    o1, m1 = KV.decode_step(q, m.pool.numpy(), m.table_host, m.lens, 0.0883)
    o2, m2 = OA.decode_step(q, m.pool.numpy(), m.table_host, m.lens, 0.0883)
    assert np.array_equal(o1, o2)
    assert all(np.array_equal(a, b) for a, b in zip(m1, m2))


@pytest.mark.parametrize("n", [160, 300])
def test_kivi_kv_quantises_exactly_the_boundary(n):
    rng = np.random.default_rng(n)
    K = _f16(rng.standard_normal((n, 128)))
    V = _f16(rng.standard_normal((n, 128)))
    Kh, Vh = KV.kivi_kv(K, V, n)
    nq = KV.quant_boundary(n)
    assert np.array_equal(Kh[nq:], K[nq:].astype(np.float64))
    assert np.array_equal(Vh[nq:], V[nq:].astype(np.float64))
    assert np.all(np.any(Kh[:nq] != K[:nq].astype(np.float64), axis=1))
