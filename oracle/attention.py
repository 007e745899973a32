"""Dense decode attention over a paged KV cache, in fp64, plus block mass.

What one decode step computes, written as its plain definition:

1. Gather.  Token t of sequence s lives in physical block
   table[s][t // 16] at slot t % 16 (KV cache offload post, "Top row": the
   per-sequence block table maps logical positions to physical block ids).
   A physical block holds every layer, K and V, all 8 KV heads (GQA Per-Head
   Scoring Streams: the block travels with all KV heads of all layers).
2. Attention.  The new token's query of head h attends over every position
   of its sequence (Visual Reference Sec. 4, Diagram 4.1: decode reads the
   entire cache) with the key/value of KV head g = h // 8 (GQA Per-Head
   Scoring Streams, panel 1: Q0-Q7 -> KV-head 0, ..., Q56-Q63 -> KV-head 7):
   z_t = scale * <q_h, k_t>, p = softmax(z), out_h = sum_t p_t v_t
   (Visual Reference Sec. 2, Diagram 2.2: scores, softmax, weighted sum of V).
   No causal mask: the query is the newest position.  No position encoding
   is applied (the synthetic q and k stand for post-rotation vectors).
3. Block mass.  The 640 (layer, KV-head) streams -- each the 8 query heads
   of its group -- are aggregated into one number per (sequence, block)
   (GQA Per-Head Scoring Streams, panel 2).  The page names no operator; the
   reading used here is the sum of softmax probability over every layer in
   range, every query head and every token of the block.

Parity pins (tests/test_oracle_attention.py): q = 0 gives uniform
probabilities and out = mean(V); a one-hot key gives a closed-form weight;
a pure-Python loop on tiny inputs; torch's fp64 scaled_dot_product_attention
on an independently gathered, head-repeated K/V; bit-identical output under
a permutation of physical placement; the GQA group map; mass sums.
"""
from __future__ import annotations

import numpy as np

from . import fp8

BLOCK_TOKENS = 16
GROUP = 8  # query heads per KV head


def _values(raw, kv_format: str):
    """Stored K/V elements to fp64: fp16 values, or E4M3 codes (uint8)."""
    if kv_format == "fp16":
        return np.asarray(raw, dtype=np.float64)
    if kv_format == "e4m3":
        return fp8.decode_pool(raw)
    raise ValueError(f"unknown KV format {kv_format}")


def gather_layer(pool, table_row, n_tokens: int, layer: int, kv_head=None,
                 kv_format: str = "fp16"):
    """K and V of one sequence at one layer, fp64.

    pool:      array [P][L][2][H_kv][16][D] of fp16 values or E4M3 codes,
               indexable with numpy ints.
    table_row: physical block id of each logical block.
    Returns K, V shaped [H_kv][n][D] (or [n][D] when kv_head is given).
    """
    nb = -(-n_tokens // BLOCK_TOKENS)
    pids = np.asarray(table_row[:nb], dtype=np.int64)
    if kv_head is None:
        blocks = _values(pool[pids, layer], kv_format)                  # [nb][2][H][16][D]
        kv = blocks.transpose(1, 2, 0, 3, 4)                           # [2][H][nb][16][D]
        kv = kv.reshape(2, kv.shape[1], nb * BLOCK_TOKENS, kv.shape[-1])[:, :, :n_tokens]
        return kv[0], kv[1]
    blocks = _values(pool[pids, layer, :, kv_head], kv_format)            # [nb][2][16][D]
    kv = blocks.transpose(1, 0, 2, 3).reshape(2, nb * BLOCK_TOKENS, blocks.shape[-1])
    return kv[0, :n_tokens], kv[1, :n_tokens]


def attend_head(q_h, K_g, V_g, scale: float):
    """Softmax attention of one query row over one KV head's tokens.

    Returns (out [D], p [n]) in fp64.
    """
    z = scale * (K_g @ np.asarray(q_h, dtype=np.float64))
    z = z - z.max()
    e = np.exp(z)
    p = e / e.sum()
    return p @ V_g, p


def block_sums(p, n_tokens: int):
    """Sum of p over each 16-token block (the last block may be partial)."""
    nb = -(-n_tokens // BLOCK_TOKENS)
    padded = np.zeros(nb * BLOCK_TOKENS, dtype=np.float64)
    padded[:n_tokens] = p
    return padded.reshape(nb, BLOCK_TOKENS).sum(axis=1)


def decode_layer(q_sl, pool, table_row, n_tokens: int, layer: int, scale: float,
                 kv_format: str = "fp16"):
    """All 64 query heads of one (sequence, layer).

    Returns out [64][D] fp64 and the block mass of this layer [nb] fp64.
    """
    if n_tokens == 0:   # an empty sequence attends to nothing: zero output, no blocks
        return np.zeros((q_sl.shape[0], q_sl.shape[-1]), dtype=np.float64), np.zeros(0)
    K, V = gather_layer(pool, table_row, n_tokens, layer, kv_format=kv_format)
    n_q = q_sl.shape[0]
    out = np.empty((n_q, K.shape[-1]), dtype=np.float64)
    mass = np.zeros(-(-n_tokens // BLOCK_TOKENS), dtype=np.float64)
    for h in range(n_q):
        g = h // GROUP
        out[h], p = attend_head(q_sl[h], K[g], V[g], scale)
        mass += block_sums(p, n_tokens)
    return out, mass


def decode_step(q, pool, block_table, seq_lens, scale: float,
                layer_begin: int = 0, layer_end=None, kv_format: str = "fp16"):
    """One decode step for a batch.

    q: [B][L][64][D]; pool: [P][L][2][8][16][D]; block_table: [B][max_nb];
    seq_lens: [B] token counts; kv_format: "fp16" (pool holds values) or
    "e4m3" (pool holds E4M3 codes, Fitting a Million Tokens Sec. 02).
    Returns out [B][L][64][D] fp64 (NaN outside [layer_begin, layer_end)) and a
    list with one fp64 array [nb_s] of block mass per sequence, summed over the
    layers in range and all query heads.
    """
    q = np.asarray(q)
    B, L = q.shape[0], q.shape[1]
    if layer_end is None:
        layer_end = L
    out = np.full(q.shape, np.nan, dtype=np.float64)
    masses = []
    for s in range(B):
        n = int(seq_lens[s])
        mass = np.zeros(-(-n // BLOCK_TOKENS), dtype=np.float64)
        for layer in range(layer_begin, layer_end):
            out[s, layer], m = decode_layer(q[s, layer], pool, block_table[s], n, layer, scale,
                                            kv_format)
            mass += m
        masses.append(mass)
    return out, masses
