"""Device-memory plumbing around the C ABI for one materialised workload.

Allocates (with torch) the output, block-mass, record and workspace buffers a
decode + scoring step needs, and calls the library.  No arithmetic here; for
a KIVI cache it asks the library which tokens are quantised (its window rule,
kvs_kivi_quant_len) and places the quantised blocks.
"""
from __future__ import annotations

import numpy as np
import torch

import workload as W

from . import api


def pair_plan(table_host, blocks) -> np.ndarray:
    """pair_role for kvs_decode_step_paired: sequences whose first block is the
    same physical block (a shared prefix), paired in batch order; -1 for the
    rest.  Only a plan: the decode is bit-identical with or without it."""
    B = len(blocks)
    role = np.full(B, -1, dtype=np.int32)
    groups = {}
    for s in range(B):
        if blocks[s] > 0:
            groups.setdefault(int(table_host[s, 0]), []).append(s)
    for members in groups.values():
        for a, b in zip(members[0::2], members[1::2]):
            role[a] = b
            role[b] = -2 - a
    return role


def pair_loaded_tokens(table_host, lens, role, split_blocks: int) -> int:
    """Tokens whose keys and values the paired decode loads per (layer, KV
    head).  A split is joint when its two sequences are linked both ways, both
    reach the split's first position and hold the same block there.  A joint
    split walks its positions one block at a time: a position where the two
    sequences hold the same block (or only one of them reaches) is loaded
    once, for the larger of the two token counts, any other position once per
    sequence.  Every other split loads its own sequence's tokens, as the
    unpaired decode does."""
    role = np.asarray(role)
    B, SB = len(lens), int(split_blocks)
    lens = np.asarray(lens, dtype=np.int64)
    nb = (lens + 15) // 16
    tbl = table_host

    def link_of(s):   # (first, second) of s's mutual link, or None
        o = int(role[s])
        other = o if o >= 0 else -2 - o
        if o == -1 or other == s or not 0 <= other < B:
            return None
        if o >= 0 and int(role[other]) == -2 - s:
            return s, other
        if o <= -2 and int(role[other]) == s:
            return other, s
        return None

    def tokens_at(s, b, b1):
        return int(min(16, lens[s] - 16 * b)) if b < b1 else 0

    tokens = 0
    for s in range(B):
        link = link_of(s)
        for b0 in range(0, int(nb[s]), SB):
            b1 = min(int(nb[s]), b0 + SB)
            joint = (link is not None and b0 < nb[link[0]] and b0 < nb[link[1]]
                     and tbl[link[0], b0] == tbl[link[1], b0])
            if not joint:
                tokens += int(min(lens[s], 16 * b1) - 16 * b0)
                continue
            if link[0] != s:
                continue   # loaded by the first sequence's work-groups
            p = link[1]
            b1p = min(int(nb[p]), b0 + SB)
            for b in range(b0, max(b1, b1p)):
                same = not (b < b1 and b < b1p and tbl[s, b] != tbl[p, b])
                va, vb = tokens_at(s, b, b1), tokens_at(p, b, b1p)
                tokens += max(va, vb) if same else va + vb
    return tokens


class DecodeSession:
    def __init__(self, m, layer_begin: int = 0, layer_end=None, split_blocks: int = 0,
                 anchor_blocks: int = 1, stream=None, kivi_spare_blocks=None, pair_role=None):
        self.m = m
        self.stream = stream
        L = m.num_layers
        self.layer_begin = layer_begin
        self.layer_end = L if layer_end is None else layer_end
        self.shape = api.shape(L)
        dev = m.pool.device
        B = m.batch
        fmt = m.workload.kv_format
        self.kv_format = fmt
        self.split_blocks = api.decode_split_blocks(self.shape, B, m.max_blocks, self.layer_begin,
                                                    self.layer_end, split_blocks, fmt)
        if self.split_blocks == 0:
            raise ValueError(f"invalid split_blocks {split_blocks}")
        # paired decode (fp16, E4M3): pair_role as kvs_decode_step_paired takes
        # it, or "auto" for pair_plan's shared-prefix pairs; automatic splits of
        # at most 512 blocks (fp16) or 256 (E4M3)
        self.pair_role = None
        if pair_role is not None:
            if fmt not in ("fp16", "e4m3"):
                raise ValueError("paired decode runs over fp16 or E4M3 pools only")
            if isinstance(pair_role, str) and pair_role == "auto":
                pair_role = pair_plan(m.table_host, m.blocks)
            self.pair_role = torch.as_tensor(np.asarray(pair_role, dtype=np.int32), device=dev)
            if split_blocks == 0:   # the library's automatic choice for pairs
                self.split_blocks = min(self.split_blocks, 256 if fmt == "e4m3" else 512)
        self.out = torch.zeros((B, L, 64, 128), dtype=torch.float16, device=dev)
        self.mass = torch.zeros(max(m.total_blocks, 1), dtype=torch.float32, device=dev)
        ws_bytes = api.decode_workspace_bytes(self.shape, B, m.max_blocks, m.total_blocks,
                                              self.layer_begin, self.layer_end, self.split_blocks,
                                              fmt)
        self.ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        api.workspace_init(self.ws, stream=stream)
        self.meta = torch.empty((max(m.total_blocks, 1), 64), dtype=torch.uint8, device=dev)
        self.score_ws = torch.empty(api.score_workspace_bytes(B, m.max_blocks), dtype=torch.uint8,
                                    device=dev)
        api.workspace_init(self.score_ws, stream=stream)
        self.anchor_blocks = anchor_blocks
        self.reset_meta()
        if fmt == "kivi2":
            self._build_kivi(8 * B if kivi_spare_blocks is None else kivi_spare_blocks)

    def _build_kivi(self, spare: int):
        """Quantise every sequence's tokens below its KIVI boundary with the
        library's quantiser into a separate pool of quantised blocks, and point
        those table entries at it.  Pairs of fp16 blocks shared between
        sequences are quantised once."""
        m = self.m
        dev = m.pool.device
        table = m.table_host
        self.quant_lens_host = np.array([api.kivi_quant_len(n) for n in m.lens], dtype=np.int32)
        pairs, where = [], {}
        kivi_table = table.astype(np.int32).copy()
        for s_ in range(m.batch):
            for p in range(int(self.quant_lens_host[s_]) // 32):
                src = (int(table[s_, 2 * p]), int(table[s_, 2 * p + 1]))
                if src not in where:
                    where[src] = len(pairs)
                    pairs.append(src)
                k = where[src]
                kivi_table[s_, 2 * p:2 * p + 2] = (2 * k, 2 * k + 1)
        n_blocks = max(2, 2 * len(pairs) + spare)
        place = W.kivi_placement(m.workload, n_blocks)       # pair k -> blocks place[2k], place[2k+1]
        self.kivi_free_host = place[2 * len(pairs):].copy()  # quantised blocks not in use
        for s_ in range(m.batch):
            nqb = int(self.quant_lens_host[s_]) // 16
            kivi_table[s_, :nqb] = place[kivi_table[s_, :nqb]]
        spec = np.zeros((max(1, len(pairs)), 4), dtype=np.int32)
        for k, (e, o) in enumerate(pairs):
            spec[k] = (e, o, place[2 * k], place[2 * k + 1])
        self.kivi_blocks = n_blocks
        self.kivi_pool = torch.empty((n_blocks, api.kivi_block_bytes(self.shape)),
                                     dtype=torch.uint8, device=dev)
        self.kivi_table = torch.from_numpy(kivi_table).to(dev)
        self.kivi_table_host = kivi_table
        self.quant_lens = torch.from_numpy(self.quant_lens_host).to(dev)
        self.kivi_pairs = torch.from_numpy(spec).to(dev)
        self.kivi_ws = torch.empty(256, dtype=torch.uint8, device=dev)
        api.workspace_init(self.kivi_ws, stream=self.stream)
        api.kivi_quantize(self.shape, m.pool, m.pool_blocks, self.kivi_pool, n_blocks,
                          self.kivi_pairs, len(pairs), self.kivi_ws, stream=self.stream)

    @property
    def kv_elem_bytes(self) -> int:
        return 1 if self.m.workload.kv_format == "e4m3" else 2

    @property
    def kv_bytes_per_step(self) -> int:
        """Stored KV bytes one decode step reads (keys and values, every token of
        the lengths materialised; appends grow this by one token per sequence).
        Under KIVI: 768-byte tiles for quantised blocks, fp16 for the rest."""
        layers = self.layer_end - self.layer_begin
        if self.kv_format == "kivi2":
            nq = int(self.quant_lens_host.sum())
            return (nq // 16 * 2 * 768 + (sum(self.m.lens) - nq) * 128 * 2 * 2) * layers * 8
        return sum(self.m.lens) * layers * 8 * 128 * 2 * self.kv_elem_bytes

    @property
    def kv_bytes_loaded_per_step(self) -> int:
        """Stored KV bytes the decode kernels load per step: kv_bytes_per_step,
        less what a pairing shares (pair_loaded_tokens)."""
        if self.pair_role is None:
            return self.kv_bytes_per_step
        m = self.m
        tokens = pair_loaded_tokens(m.table_host, m.lens, self.pair_role.cpu().numpy(),
                                    self.split_blocks)
        layers = self.layer_end - self.layer_begin
        return tokens * layers * 8 * 128 * 2 * self.kv_elem_bytes

    def reset_meta(self):
        m = self.m
        api.meta_init(self.meta, m.meta_offsets, m.seq_ids, m.batch, m.max_blocks, m.total_blocks,
                      self.anchor_blocks, stream=self.stream)

    def decode(self, q, accumulate: int = 0, layer_begin=None, layer_end=None, scale=None):
        m = self.m
        lb = self.layer_begin if layer_begin is None else layer_begin
        le = self.layer_end if layer_end is None else layer_end
        sc = api.DEFAULT_SCALE if scale is None else scale
        if self.kv_format == "kivi2":
            api.decode_step_kivi(self.shape, q, m.pool, m.pool_blocks, self.kivi_pool,
                                 self.kivi_blocks, self.kivi_table, m.max_blocks, m.seq_lens,
                                 self.quant_lens, m.meta_offsets, m.batch, m.total_blocks, lb, le,
                                 sc, self.out, self.mass, accumulate, self.split_blocks, self.ws,
                                 stream=self.stream)
            return
        if self.pair_role is not None:
            fn = api.decode_step_e4m3_paired if self.kv_format == "e4m3" else api.decode_step_paired
            fn(self.shape, q, m.pool, m.pool_blocks, m.block_table, m.max_blocks, m.seq_lens,
               self.pair_role, m.meta_offsets, m.batch, m.total_blocks, lb, le, sc, self.out,
               self.mass, accumulate, self.split_blocks, self.ws, stream=self.stream)
            return
        fn = api.decode_step_e4m3 if self.kv_format == "e4m3" else api.decode_step
        fn(self.shape, q, m.pool, m.pool_blocks, m.block_table, m.max_blocks, m.seq_lens,
           m.meta_offsets, m.batch, m.total_blocks, lb, le, sc, self.out, self.mass, accumulate,
           self.split_blocks, self.ws, stream=self.stream)

    def score(self, step: int, pol, classify: int = 1):
        m = self.m
        api.score_update(self.meta, self.mass, m.meta_offsets, m.seq_lens, m.batch,
                         m.max_blocks, m.total_blocks, step, pol, classify, self.score_ws,
                         stream=self.stream)

    def classify(self, pol, tiers_out=None):
        m = self.m
        api.classify(self.meta, m.meta_offsets, m.seq_lens, m.batch, m.max_blocks,
                     m.total_blocks, pol, tiers_out, stream=self.stream)

    def append(self, k_new, v_new):
        """Append one token per sequence (updates the pool, table, seq_lens and
        records in place; the host copies of lengths are not touched)."""
        m = self.m
        kivi = self.kv_format == "kivi2"
        if not hasattr(self, "free_stack"):
            dev = self.out.device
            # capacity for every pool id: a KIVI cache returns fp16 blocks to this stack
            stack = np.full(max(m.pool_blocks, 1), -1, dtype=np.int32)
            stack[:m.free_stack.size] = m.free_stack
            self.free_stack = torch.from_numpy(stack).to(dev)
            self.free_top = torch.tensor([int(m.free_stack.size)], dtype=torch.int32, device=dev)
            self.append_ws = torch.empty(api.append_workspace_bytes(m.batch), dtype=torch.uint8,
                                         device=dev)
            api.workspace_init(self.append_ws, stream=self.stream)
            if kivi:
                self.kivi_free = torch.from_numpy(self.kivi_free_host.astype(np.int32)).to(dev)
                self.kivi_free_top = torch.tensor([int(self.kivi_free_host.size)],
                                                  dtype=torch.int32, device=dev)
                self.advance_ws = torch.empty(api.kivi_advance_workspace_bytes(m.batch),
                                              dtype=torch.uint8, device=dev)
                api.workspace_init(self.advance_ws, stream=self.stream)
        eb = 1 if m.workload.kv_format == "e4m3" else 2
        table = self.kivi_table if kivi else m.block_table
        api.append_kv(self.shape, eb, k_new, v_new, m.pool, m.pool_blocks, table,
                      m.max_blocks, m.seq_lens, self.free_stack, int(self.free_stack.numel()),
                      self.free_top, self.meta, m.meta_offsets, m.seq_ids, self.anchor_blocks,
                      m.batch, m.total_blocks, self.append_ws, stream=self.stream)
        if kivi:
            # quantise the pair that left the fp16 window, if any, and free its fp16 blocks
            api.kivi_advance(self.shape, m.pool, m.pool_blocks, self.kivi_pool, self.kivi_blocks,
                             table, m.max_blocks, m.seq_lens, self.quant_lens, m.batch,
                             api.KIVI_RESIDUAL_TOKENS,
                             self.kivi_free, int(self.kivi_free.numel()), self.kivi_free_top,
                             self.free_stack, int(self.free_stack.numel()), self.free_top,
                             self.advance_ws, stream=self.stream)

    def evict_candidates(self, now: int, alpha: float, active=None, exclude_pinned: int = 0):
        """(out_block int32 [B], out_key float64 [B]) device tensors."""
        m = self.m
        if not hasattr(self, "evict_ws"):
            self.evict_ws = torch.empty(api.evict_workspace_bytes(m.batch, m.max_blocks),
                                        dtype=torch.uint8, device=self.out.device)
            api.workspace_init(self.evict_ws, stream=self.stream)
        blk = torch.empty(m.batch, dtype=torch.int32, device=self.out.device)
        key = torch.empty(m.batch, dtype=torch.float64, device=self.out.device)
        api.evict_candidates(self.meta, m.meta_offsets, m.seq_lens, active, m.batch, m.max_blocks,
                             m.total_blocks, now, alpha, exclude_pinned, blk, key, self.evict_ws,
                             stream=self.stream)
        return blk, key

    def step(self, q, step: int, pol, classify: int = 1):
        self.decode(q)
        self.score(step, pol, classify)

    def status(self) -> int:
        bits = api.device_status(self.ws, self.stream) | api.device_status(self.score_ws, self.stream)
        if hasattr(self, "evict_ws"):
            bits |= api.device_status(self.evict_ws, self.stream)
        if hasattr(self, "append_ws"):
            bits |= api.device_status(self.append_ws, self.stream)
        if hasattr(self, "kivi_ws"):
            bits |= api.device_status(self.kivi_ws, self.stream)
        if hasattr(self, "advance_ws"):
            bits |= api.device_status(self.advance_ws, self.stream)
        return bits

    def records(self):
        return api.records(self.meta[: self.m.total_blocks])
