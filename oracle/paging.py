"""Appending the new token's K/V to a paged cache, with block allocation.

Generation adds one key and one value per layer per KV head for every new
token (Fitting a Million Tokens, Sec. 01: the per-token KV cost).  The cache
is paged: fixed 16-token blocks, a per-sequence table of physical block ids,
blocks taken from and returned to a pool by a block manager (KV cache
offload post, "Top row").  One append step, for every sequence s in batch
order:

* the new token's position is t = n_s (the sequence's current length); it goes
  to logical block b = t // 16 at slot t % 16;
* when t % 16 == 0 the sequence needs a new physical block: blocks are taken
  from the top of a free-block stack, sequences in batch order (the first
  sequence needing one takes free[top - 1], the next free[top - 2], ...); the
  table entry table[s][b] is set and the block's record is created fresh
  (score 0, never touched, unclassified);
* K and V of the token are written to that slot for every layer and KV head;
  nothing else in the pool changes (a written slot is never rewritten);
* n_s grows by one.

A sequence that needs a block when the stack is empty, or whose table row is
full, is left unchanged and reported.

This module keeps its own copies (NumPy) and is written for clarity, not
speed.  Parity pins (tests/test_oracle_paging.py): the appended token reads
back exactly through the gather; every earlier token is unchanged; allocation
order, stack accounting and exhaustion; lengths crossing block boundaries.
"""
from __future__ import annotations

import numpy as np

BLOCK_TOKENS = 16


def append_step(pool, table, seq_lens, free_stack, free_top: int, k_new, v_new):
    """One append over the batch.

    pool:       [P][L][2][8][16][D] array (values or codes), modified in place.
    table:      [B][max_nb] int array, modified in place.
    seq_lens:   [B] int array, modified in place.
    free_stack: [F] int array of free physical ids; entries [0, free_top) are free.
    k_new, v_new: [B][L][8][D], in the pool's storage format.
    Returns (new free_top, list of (s, b, pid) allocations, list of rejected s).
    """
    B = table.shape[0]
    max_nb = table.shape[1]
    allocs = []
    rejected = []
    for s in range(B):
        t = int(seq_lens[s])
        b, slot = divmod(t, BLOCK_TOKENS)
        if slot == 0:
            if b >= max_nb or free_top == 0:
                rejected.append(s)
                continue
            free_top -= 1
            pid = int(free_stack[free_top])
            table[s, b] = pid
            allocs.append((s, b, pid))
        else:
            pid = int(table[s, b])
        pool[pid, :, 0, :, slot, :] = k_new[s]
        pool[pid, :, 1, :, slot, :] = v_new[s]
        seq_lens[s] = t + 1
    return free_top, allocs, rejected
