"""KIVI-style 2-bit KV cache: asymmetric quantisation plus an fp16 residual window.

Test infrastructure: only tests/, the smoke check and bench.py's CPU baseline
use this module; it shares no code with the HIP library.

What the method computes (Fitting a Million Tokens, Sec. 02, "Quantize the
cache", the KIVI paragraphs and the effective-bits note):

* Asymmetric quantisation of a group of G = 32 elements to B = 2 bits: the
  group's minimum is the zero point z, the step is s = (max - min) / (2^B - 1),
  element x gets the code round((x - z) / s) in [0, 3], and reads back as
  z + code * s.  Scale and zero point are stored in fp16, one pair per group,
  so 2-bit codes cost about 3 bits per element.
* Keys are grouped per channel, along the token axis: one group is one channel
  over 32 consecutive tokens, i.e. over two 16-token blocks.  Values are
  grouped per token, along the channel axis: one group is 32 consecutive
  channels of one token.
* The newest tokens stay in fp16 (a residual window of about 128 tokens); the
  boundary between quantised and fp16 tokens is snapped down to a multiple of
  the group size, so every quantised key group holds 32 tokens.

Readings where the section leaves a step open (same on both sides):
* window and boundary: n_q = max(0, floor((n - 128) / 32) * 32) tokens of a
  sequence of n tokens are quantised; tokens [n_q, n) stay fp16 (128 to 159
  of them once n >= 160);
* arithmetic of the code decision: z = min (an fp16 value, kept exactly);
  s = fp16( fp32( fp32(max - min) / 3 ) ) (round to nearest even at each
  step); code = clamp(rint(fp32(fp32(x - z) / s)), 0, 3) with the fp16 s;
  a group whose s is 0 (all elements equal, or a span below fp16's range)
  stores code 0 everywhere;
* read-back value: z + code * s exactly (no further rounding);
* inputs are finite fp16 values.

The packed storage format of quantised blocks (the bytes the HIP library
writes and reads) is defined in `pack_k_tile` / `pack_v_tile` below, from the
description in include/kvs.h; the tests use it to read the library's output.

Parity pins (tests/test_oracle_kivi.py): values on an exact 4-level grid
round-trip exactly; the read-back error of random groups is within half a
step; equal elements give scale 0 and exact read-back; brute-force loops over
a tiny tensor give the same groups, scales and codes (keys per channel over
tokens, values per token over channels); an outlier channel stays confined to
its own key groups; the boundary rule on hand-computed lengths; the effective
bits and compression ratio the section prints; hand-placed bits of the packed
format and pack/unpack round trips; decode over a losslessly quantisable cache
equals the fp16 decode, and sequences shorter than 160 tokens are untouched.
"""
from __future__ import annotations

import numpy as np

from . import attention as OA

GROUP = 32           # elements per quantisation group (keys: tokens, values: channels)
LEVELS = 4           # 2-bit codes
RESIDUAL = 128       # fp16 residual window (tokens)
HEAD_DIM = 128
BLOCK_TOKENS = 16
TILE_BYTES = 768     # one (layer, K|V, KV head) tile of a quantised block


def quant_boundary(n: int, residual: int = RESIDUAL, group: int = GROUP) -> int:
    """Tokens [0, n_q) of an n-token sequence are quantised, [n_q, n) stay fp16."""
    return max(0, (int(n) - residual) // group * group)


def quantize_groups(x, axis: int):
    """Asymmetric 2-bit quantisation of fp16 groups lying along `axis`.

    x: fp16 array whose extent along `axis` is one group.  Returns codes
    (uint8, same shape as x), scale and zero (fp16, `axis` removed).
    """
    x = np.asarray(x, dtype=np.float16)
    x32 = x.astype(np.float32)
    lo = x32.min(axis=axis)
    hi = x32.max(axis=axis)
    span = (hi - lo).astype(np.float32)
    s16 = (span / np.float32(LEVELS - 1)).astype(np.float32).astype(np.float16)
    s32 = np.expand_dims(s16.astype(np.float32), axis)
    z32 = np.expand_dims(lo, axis)
    diff = (x32 - z32).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (diff / np.where(s32 == 0, np.float32(1), s32)).astype(np.float32)
    codes = np.clip(np.rint(t), 0, LEVELS - 1)
    codes = np.where(s32 == 0, 0, codes).astype(np.uint8)
    return codes, s16, lo.astype(np.float16)


def dequantize(codes, scale, zero, axis: int):
    """z + code * s in fp64, with scale and zero broadcast along `axis`."""
    s = np.expand_dims(np.asarray(scale, dtype=np.float64), axis)
    z = np.expand_dims(np.asarray(zero, dtype=np.float64), axis)
    return z + np.asarray(codes, dtype=np.float64) * s


def quantize_keys(K):
    """K: fp16 [n][D] with n a multiple of 32.  Per channel, groups of 32 tokens.

    Returns codes [n][D], scale [n/32][D], zero [n/32][D].
    """
    K = np.asarray(K, dtype=np.float16)
    n, d = K.shape
    assert n % GROUP == 0
    g = K.reshape(n // GROUP, GROUP, d)                    # [group][token in group][channel]
    codes, s, z = quantize_groups(g, axis=1)
    return codes.reshape(n, d), s, z


def quantize_values(V):
    """V: fp16 [n][D].  Per token, groups of 32 channels.

    Returns codes [n][D], scale [n][D/32], zero [n][D/32].
    """
    V = np.asarray(V, dtype=np.float16)
    n, d = V.shape
    g = V.reshape(n, d // GROUP, GROUP)                    # [token][group][channel in group]
    codes, s, z = quantize_groups(g, axis=2)
    return codes.reshape(n, d), s, z


def dequantize_keys(codes, s, z):
    n, d = codes.shape
    return dequantize(codes.reshape(n // GROUP, GROUP, d), s, z, axis=1).reshape(n, d)


def dequantize_values(codes, s, z):
    n, d = codes.shape
    return dequantize(codes.reshape(n, d // GROUP, GROUP), s, z, axis=2).reshape(n, d)


def kivi_kv(K, V, n: int):
    """What a KIVI cache holds for one (sequence, layer, KV head), read back.

    K, V: fp16 [>= n][D] originals.  Returns fp64 K_hat, V_hat [n][D]: tokens
    below the boundary quantised and read back, the residual window exact.
    """
    nq = quant_boundary(n)
    K = np.asarray(K[:n], dtype=np.float16)
    V = np.asarray(V[:n], dtype=np.float16)
    Kh = K.astype(np.float64)
    Vh = V.astype(np.float64)
    if nq:
        Kh[:nq] = dequantize_keys(*quantize_keys(K[:nq]))
        Vh[:nq] = dequantize_values(*quantize_values(V[:nq]))
    return Kh, Vh


def decode_layer(q_sl, pool, table_row, n: int, layer: int, scale: float):
    """All 64 query heads of one (sequence, layer) over its KIVI cache.

    Returns out [64][D] fp64 and the block mass of this layer [nb] fp64.
    """
    if n == 0:          # an empty sequence attends to nothing: zero output, no blocks
        return np.zeros((q_sl.shape[0], HEAD_DIM), dtype=np.float64), np.zeros(0)
    K16, V16 = _gather16(pool, table_row, n, layer)
    out = np.empty((q_sl.shape[0], HEAD_DIM), dtype=np.float64)
    mass = np.zeros(-(-n // BLOCK_TOKENS), dtype=np.float64)
    for g in range(8):
        Kh, Vh = kivi_kv(K16[g], V16[g], n)
        for h in range(8 * g, 8 * g + 8):
            out[h], p = OA.attend_head(q_sl[h], Kh, Vh, scale)
            mass += OA.block_sums(p, n)
    return out, mass


def decode_step(q, pool, block_table, seq_lens, scale: float, layer_begin: int = 0,
                layer_end=None):
    """One decode step over KIVI caches built from an fp16 pool.

    Same arguments and results as attention.decode_step with kv_format fp16,
    except that every (sequence, layer, KV head) stream is first replaced by
    what its KIVI cache reads back (kivi_kv).
    """
    q = np.asarray(q)
    B, L = q.shape[0], q.shape[1]
    if layer_end is None:
        layer_end = L
    out = np.full(q.shape, np.nan, dtype=np.float64)
    masses = []
    for s in range(B):
        n = int(seq_lens[s])
        nb = -(-n // BLOCK_TOKENS)
        mass = np.zeros(nb, dtype=np.float64)
        for layer in range(layer_begin, layer_end):
            out[s, layer], ms = decode_layer(q[s, layer], pool, block_table[s], n, layer, scale)
            mass += ms
        masses.append(mass)
    return out, masses


def _gather16(pool, table_row, n: int, layer: int):
    """fp16 K, V [8][n][D] of one sequence and layer (no conversion)."""
    nb = -(-n // BLOCK_TOKENS)
    pids = np.asarray(table_row[:nb], dtype=np.int64)
    blocks = np.asarray(pool[pids, layer])                             # [nb][2][8][16][D]
    kv = blocks.transpose(1, 2, 0, 3, 4).reshape(2, blocks.shape[2], nb * BLOCK_TOKENS, -1)
    return kv[0, :, :n], kv[1, :, :n]


# ---------------------------------------------------------------------------
# Packed storage of quantised blocks (the library's format, include/kvs.h).
#
# A quantised block holds, per layer, 8 key tiles then 8 value tiles of 768
# bytes (one per KV head).  Bytes [0, 512) of a tile are the 2-bit codes of
# the block's 16 tokens x 128 channels as 64 little-endian 8-byte entries,
# entry l = 16 j + c (j = l // 16, c = l % 16).  An entry is two 32-bit words
# holding four sets S = 0..3 of 8 codes: set S lives in word S // 2, code m of
# the set at bits 4 m + 2 (S % 2) of that word.
#   key tile:   entry (j, c) holds token c; set S = i holds channels
#               32 i + 8 j + m, m = 0..7.
#   value tile: entry (j, c) holds channel group c of each 16-channel tile;
#               set S holds tiles k = 2 S and 2 S + 1; code m = 4 (k % 2) + r
#               is token 4 j + r of channel 16 k + c.
# Bytes [512, 768): group parameters, fp16, 128 bytes of scales then 128
# bytes of zero points.
#   key tile:   64 channels: channels 0..63 in the even block of a 32-token
#               pair, 64..127 in the odd block; channel d's scale at
#               512 + 2 (d % 64), its zero point at 640 + 2 (d % 64).
#   value tile: token t, channel group g: scale at 512 + 2 (16 g + t), zero
#               point at 640 + 2 (16 g + t).
# ---------------------------------------------------------------------------

def _set_base(S):
    """Bit offset, inside a 64-bit entry, of code 0 of set S (code m is 4 m further)."""
    return 32 * (S // 2) + 2 * (S % 2)


def pack_codes(entry_codes):
    """entry_codes: uint8 [64][4][8] (entry, set, m) -> 512 bytes."""
    out = np.zeros(64, dtype=np.uint64)
    ec = np.asarray(entry_codes, dtype=np.uint64)
    for S in range(4):
        base = _set_base(S)
        for m in range(8):
            out |= (ec[:, S, m] & np.uint64(3)) << np.uint64(base + 4 * m)
    return out.astype("<u8").tobytes()


def unpack_codes(raw):
    """512 bytes -> uint8 [64][4][8] (entry, set, m)."""
    w = np.frombuffer(bytes(raw), dtype="<u8").astype(np.uint64)
    out = np.zeros((64, 4, 8), dtype=np.uint8)
    for S in range(4):
        base = _set_base(S)
        for m in range(8):
            out[:, S, m] = ((w >> np.uint64(base + 4 * m)) & np.uint64(3)).astype(np.uint8)
    return out


def k_entry_layout():
    """(token, channel) of every (entry, set, m) of a key tile: int arrays [64][4][8]."""
    e = np.arange(64)[:, None, None]
    S = np.arange(4)[None, :, None]
    m = np.arange(8)[None, None, :]
    j, c = e // 16, e % 16
    return np.broadcast_to(c, (64, 4, 8)), 32 * S + 8 * j + m


def v_entry_layout():
    """(token, channel) of every (entry, set, m) of a value tile: int arrays [64][4][8]."""
    e = np.arange(64)[:, None, None]
    S = np.arange(4)[None, :, None]
    m = np.arange(8)[None, None, :]
    j, c = e // 16, e % 16
    k = 2 * S + m // 4
    r = m % 4
    return np.broadcast_to(4 * j + r, (64, 4, 8)), 16 * k + c


def pack_k_tile(codes16, scale, zero, odd: bool) -> bytes:
    """codes16: uint8 [16][128] of one block; scale, zero: fp16 [128] of the
    32-token group the block belongs to; odd: the block is the second of the pair."""
    t, d = k_entry_layout()
    raw = pack_codes(np.asarray(codes16)[t, d])
    half = slice(64, 128) if odd else slice(0, 64)
    return (raw + np.asarray(scale, np.float16)[half].astype("<f2").tobytes()
            + np.asarray(zero, np.float16)[half].astype("<f2").tobytes())


def pack_v_tile(codes16, scale, zero) -> bytes:
    """codes16: uint8 [16][128]; scale, zero: fp16 [16][4] (token, channel group)."""
    t, d = v_entry_layout()
    raw = pack_codes(np.asarray(codes16)[t, d])
    planes = [np.asarray(a, np.float16).T.astype("<f2").tobytes() for a in (scale, zero)]
    return raw + planes[0] + planes[1]


def unpack_k_tile(raw):
    """-> codes [16][128] uint8, (scale, zero) fp16 [64] for this block's half."""
    raw = bytes(raw)
    t, d = k_entry_layout()
    codes = np.zeros((16, 128), dtype=np.uint8)
    codes[t, d] = unpack_codes(raw[:512])
    meta = np.frombuffer(raw[512:768], dtype="<f2").reshape(2, 64)
    return codes, meta[0].astype(np.float16), meta[1].astype(np.float16)


def unpack_v_tile(raw):
    """-> codes [16][128] uint8, scale [16][4], zero [16][4] fp16."""
    raw = bytes(raw)
    t, d = v_entry_layout()
    codes = np.zeros((16, 128), dtype=np.uint8)
    codes[t, d] = unpack_codes(raw[:512])
    meta = np.frombuffer(raw[512:768], dtype="<f2").reshape(2, 4, 16)
    return codes, meta[0].T.astype(np.float16), meta[1].T.astype(np.float16)


def pack_pair(K32, V32):
    """Quantise and pack one 32-token pair of one (layer, KV head).

    K32, V32: fp16 [32][128].  Returns (k_even, k_odd, v_even, v_odd) tiles.
    """
    kc, ks, kz = quantize_keys(K32)
    vc, vs, vz = quantize_values(V32)
    return (pack_k_tile(kc[:16], ks[0], kz[0], False), pack_k_tile(kc[16:], ks[0], kz[0], True),
            pack_v_tile(vc[:16], vs[:16], vz[:16]), pack_v_tile(vc[16:], vs[16:], vz[16:]))
