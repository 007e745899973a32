"""Seeded synthetic workloads: paged fp16 K/V pool, block tables, queries.

What is drawn (no step of the method is computed here):

* Head shape of the 70B-class model the pages size everything on
  (KV-Cache Offloading for LLM Inference -- Visual Reference, Sec. 1
  "Architecture Parameters"): 64 query heads, 8 KV heads, head_dim 128,
  fp16, 16-token blocks.
* Pool layout ``[pool_blocks][L][2][8][16][128]`` fp16: one physical block
  holds 16 tokens of every layer, K and V, all 8 KV heads, so the whole
  block moves as one unit (GQA Per-Head Scoring Streams, panel 2 and the
  per-block state panel; KV cache offload blog, "Top row": fixed-size
  blocks, per-sequence block table of physical ids, refcounted sharing).
* Values: q, K, V ~ N(0, 1).  One unit vector u per (layer, KV head);
  +q_boost*u is added to the 8 queries of the group and +k_boost*u to the
  keys of block 0 and of the last tenth of the positions, so that attention
  favours the anchor and the recent tail the way the appendix's locality
  section assumes (Visual Reference Sec. 6).  Rounding to fp16 happens once,
  after the addition.
* Physical placement is a seeded random permutation of the pool; pool
  blocks that no table references are filled with NaN (fp16 NaN, or the E4M3
  NaN code 0x7F) so that a stray read poisons the result.
* kv_format "e4m3" stores the same drawn values rounded once to FP8 E4M3
  codes with no scale (Fitting a Million Tokens, Sec. 02).
* kv_format "kivi2" keeps the fp16 values in the pool; the 2-bit KIVI cache
  of the same section is built from them by the consumer (the library's
  quantiser, or the oracle on the test side).  KIVI pool placement is a
  seeded permutation (kivi_placement).
* A shared prefix is expressed the paged way: the same physical ids appear
  in several tables and carry a reference count (KV cache offload blog,
  "Top row").  Shared blocks take only the block-0 boost; the recent-tail
  boost goes to a sequence's private positions only.

Host-side structure (lengths, permutation, tables) comes from NumPy's
PCG64 and is identical on every device.  Values come from torch's generator
on the target device, so the CPU and GPU draw different numbers; parity
always hands both sides the same materialised tensors.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch

NUM_Q_HEADS = 64
NUM_KV_HEADS = 8
HEAD_DIM = 128
BLOCK_TOKENS = 16
GROUP = NUM_Q_HEADS // NUM_KV_HEADS

# Blocks generated per randn call; part of the recipe (changing it changes the
# drawn values on a device).
_GEN_CHUNK_BLOCKS = 4096


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    num_layers: int
    batch: int
    steps: int
    alphas: tuple
    seed: int
    seq_lens: Optional[tuple] = None          # explicit token counts
    length_range: Optional[tuple] = None      # (lo, hi) uniform, rounded to 16
    pool_blocks: Optional[int] = None         # None: unique blocks needed + spare
    spare_blocks: int = 0
    shared_prefix_tokens: int = 0
    q_boost: float = 4.0
    k_boost: float = 0.5
    recent_den: int = 10                      # "last 1/recent_den of positions"
    kv_format: str = "fp16"                   # "fp16" values or "e4m3" codes (uint8)

    def lengths(self) -> list:
        if self.seq_lens is not None:
            assert len(self.seq_lens) == self.batch
            return [int(n) for n in self.seq_lens]
        lo, hi = self.length_range
        rng = np.random.default_rng(self.seed)
        u = rng.uniform(lo, hi, size=self.batch)
        return [int(BLOCK_TOKENS * round(x / BLOCK_TOKENS)) for x in u]


WORKLOADS = {
    # 1 layer, batch 1, 1,024 tokens = 64 blocks in a 256-block pool.
    "decode-1L-1K": Workload("decode-1L-1K", num_layers=1, batch=1, steps=10,
                             alphas=(0.15,), seed=0, seq_lens=(1024,),
                             pool_blocks=256),
    # 4 layers, 8 sequences of 8,192 tokens over a shared 8,192-block pool.
    "decode-4L-8x8K": Workload("decode-4L-8x8K", num_layers=4, batch=8, steps=32,
                               alphas=(0.15,), seed=1000, seq_lens=(8192,) * 8,
                               pool_blocks=8192),
    # 80 layers, batch 1, 131,072 tokens (8,192 blocks, 40.0 GiB of KV).
    "decode-80L-128K": Workload("decode-80L-128K", num_layers=80, batch=1, steps=16,
                                alphas=(0.05, 0.15), seed=2000,
                                seq_lens=(131072,), spare_blocks=64),
    # 80 layers, 32 sequences of 1K..32K tokens sharing a 2,048-token prefix.
    "decode-80L-32xMixed-shared2K": Workload(
        "decode-80L-32xMixed-shared2K", num_layers=80, batch=32, steps=8,
        alphas=(0.15,), seed=3000, length_range=(1024, 32768),
        shared_prefix_tokens=2048, spare_blocks=64),
    # 32 layers, batch 1, 1,048,576 tokens (65,536 blocks, 128 GiB of KV).
    "decode-32L-1M": Workload("decode-32L-1M", num_layers=32, batch=1, steps=4,
                              alphas=(0.01, 0.15), seed=4000,
                              seq_lens=(1048576,), pool_blocks=65536),
}


def custom(name: str, num_layers: int, seq_lens: Sequence[int], *, seed: int = 7,
           steps: int = 3, alphas=(0.15,), pool_blocks: Optional[int] = None,
           spare_blocks: int = 4, shared_prefix_tokens: int = 0,
           q_boost: float = 4.0, k_boost: float = 0.5, kv_format: str = "fp16") -> Workload:
    """A small ad-hoc workload with the same recipe (ragged lengths allowed)."""
    return Workload(name, num_layers=num_layers, batch=len(seq_lens), steps=steps,
                    alphas=tuple(alphas), seed=seed, seq_lens=tuple(int(n) for n in seq_lens),
                    pool_blocks=pool_blocks, spare_blocks=spare_blocks,
                    shared_prefix_tokens=shared_prefix_tokens,
                    q_boost=q_boost, k_boost=k_boost, kv_format=kv_format)


def as_e4m3(wl: Workload) -> Workload:
    """The same workload with the KV pool stored as E4M3 codes."""
    return dataclasses.replace(wl, name=wl.name + "-e4m3", kv_format="e4m3")


def as_kivi2(wl: Workload) -> Workload:
    """The same workload decoded through a KIVI 2-bit cache (fp16 pool as source)."""
    return dataclasses.replace(wl, name=wl.name + "-kivi2", kv_format="kivi2")


def kivi_placement(wl: Workload, n_blocks: int) -> np.ndarray:
    """Seeded random physical ids 0..n_blocks-1 for quantised blocks."""
    return np.random.default_rng([wl.seed, 2]).permutation(n_blocks).astype(np.int32)


@dataclasses.dataclass
class Materialised:
    workload: Workload
    pool: torch.Tensor            # fp16 [P][L][2][8][16][128]
    block_table: torch.Tensor     # int32 [B][max_blocks]; -1 past a sequence's end
    seq_lens: torch.Tensor        # int32 [B]
    meta_offsets: torch.Tensor    # int32 [B+1]; record of (s, b) is meta_offsets[s] + b
    seq_ids: torch.Tensor         # int64 [B]
    u: torch.Tensor               # fp32 [L][8][128], unit vectors
    lens: list                    # host copies
    blocks: list
    max_blocks: int
    total_blocks: int
    pool_blocks: int
    table_host: np.ndarray        # int32 [B][max_blocks]
    refcount: np.ndarray          # int32 [P]: sequences referencing each physical block
    unique_blocks: int
    free_stack: np.ndarray = None  # int32: pool blocks no table references (top = last)
    capacity: list = None          # records (and table entries) per sequence

    @property
    def num_layers(self) -> int:
        return self.workload.num_layers

    @property
    def batch(self) -> int:
        return self.workload.batch


def query_seed(seed: int, step: int) -> int:
    return (seed * 1_000_003 + 7_919 * (step + 1)) & 0x7FFF_FFFF_FFFF


def _layout(wl: Workload, extra_blocks: int = 0):
    lens = wl.lengths()
    if any(n < 0 for n in lens):
        raise ValueError("sequence lengths must be >= 0")
    blocks = [math.ceil(n / BLOCK_TOKENS) for n in lens]
    shared_nb = math.ceil(wl.shared_prefix_tokens / BLOCK_TOKENS)
    used_shared = min(shared_nb, max(blocks)) if shared_nb else 0
    unique = used_shared + sum(nb - min(nb, shared_nb) for nb in blocks)
    pool = wl.pool_blocks if wl.pool_blocks is not None else unique + wl.spare_blocks
    if pool < unique:
        raise ValueError(f"pool of {pool} blocks cannot hold {unique} unique blocks")
    rng = np.random.default_rng(wl.seed + 1)
    perm = rng.permutation(pool).astype(np.int64)
    shared = perm[:used_shared]
    cursor = used_shared
    max_nb = max(max(blocks), 1) + extra_blocks
    table = np.full((wl.batch, max_nb), -1, dtype=np.int32)
    refcount = np.zeros(pool, dtype=np.int32)
    for s, nb in enumerate(blocks):
        k = min(nb, shared_nb)
        table[s, :k] = shared[:k]
        table[s, k:nb] = perm[cursor:cursor + nb - k]
        cursor += nb - k
        np.add.at(refcount, table[s, :nb], 1)
    free = perm[cursor:].astype(np.int32)
    return lens, blocks, shared_nb, pool, table, refcount, unique, free


def _boost_positions(wl: Workload, lens, table, shared_nb):
    """Unique (physical block, slot) pairs whose keys get the +k_boost*u."""
    pairs = set()
    for s, n in enumerate(lens):
        first = range(0, min(BLOCK_TOKENS, n))
        recent_start = n - n // wl.recent_den
        private_start = min(shared_nb * BLOCK_TOKENS, n) if shared_nb else 0
        recent = range(max(recent_start, private_start), n)
        for t in list(first) + list(recent):
            pairs.add((int(table[s, t // BLOCK_TOKENS]), t % BLOCK_TOKENS))
    if not pairs:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    arr = np.array(sorted(pairs), dtype=np.int64)
    return arr[:, 0], arr[:, 1]


def materialise(wl: Workload, device="cpu", extra_blocks: int = 0) -> Materialised:
    """extra_blocks: table entries and records reserved per sequence beyond its
    current blocks, for appends; pool blocks no table references form the free
    stack."""
    device = torch.device(device)
    lens, blocks, shared_nb, pool_n, table, refcount, unique, free = _layout(wl, extra_blocks)
    L = wl.num_layers

    gen = torch.Generator(device=device)
    gen.manual_seed(wl.seed)
    u = torch.randn((L, NUM_KV_HEADS, HEAD_DIM), generator=gen, device=device,
                    dtype=torch.float32)
    u = u / u.norm(dim=-1, keepdim=True)

    if wl.kv_format not in ("fp16", "e4m3", "kivi2"):
        raise ValueError(f"unknown KV format {wl.kv_format}")
    fp8 = wl.kv_format == "e4m3"
    pool = torch.empty((pool_n, L, 2, NUM_KV_HEADS, BLOCK_TOKENS, HEAD_DIM),
                       dtype=torch.uint8 if fp8 else torch.float16, device=device)
    bp, bo = _boost_positions(wl, lens, table, shared_nb)
    bp_t = torch.from_numpy(bp).to(device)
    bo_t = torch.from_numpy(bo).to(device)
    for layer in range(L):
        gen.manual_seed(wl.seed * 1009 + 17 + layer)
        for c0 in range(0, pool_n, _GEN_CHUNK_BLOCKS):
            c1 = min(pool_n, c0 + _GEN_CHUNK_BLOCKS)
            x = torch.randn((c1 - c0, 2, NUM_KV_HEADS, BLOCK_TOKENS, HEAD_DIM),
                            generator=gen, device=device, dtype=torch.float32)
            if bp.size:
                sel = (bp_t >= c0) & (bp_t < c1)
                if bool(sel.any()):
                    pid = bp_t[sel] - c0
                    off = bo_t[sel]
                    x[pid, 0, :, off, :] += wl.k_boost * u[layer]
            if fp8:   # one rounding, straight to E4M3 (no scale)
                pool[c0:c1, layer].copy_(x.to(torch.float8_e4m3fn).view(torch.uint8))
            else:
                pool[c0:c1, layer].copy_(x.to(torch.float16))
            del x
    referenced = refcount > 0
    unused = np.nonzero(~referenced)[0]
    if unused.size:
        pool[torch.from_numpy(unused).to(device)] = 0x7F if fp8 else float("nan")

    capacity = [nb + extra_blocks for nb in blocks]
    offsets = np.zeros(wl.batch + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(capacity)
    return Materialised(
        workload=wl,
        pool=pool,
        block_table=torch.from_numpy(table).to(device),
        seq_lens=torch.tensor(lens, dtype=torch.int32, device=device),
        meta_offsets=torch.from_numpy(offsets).to(device),
        seq_ids=torch.arange(wl.batch, dtype=torch.int64, device=device),
        u=u,
        lens=lens,
        blocks=blocks,
        max_blocks=max(capacity),
        total_blocks=int(offsets[-1]),
        pool_blocks=pool_n,
        table_host=table,
        refcount=refcount,
        unique_blocks=unique,
        free_stack=free,
        capacity=capacity,
    )


def make_query(m: Materialised, step: int) -> torch.Tensor:
    """fp16 [B][L][64][128]; head h belongs to KV group h // 8."""
    wl = m.workload
    device = m.u.device
    gen = torch.Generator(device=device)
    gen.manual_seed(query_seed(wl.seed, step))
    q = torch.randn((wl.batch, wl.num_layers, NUM_KV_HEADS, GROUP, HEAD_DIM),
                    generator=gen, device=device, dtype=torch.float32)
    q += wl.q_boost * m.u[None, :, :, None, :]
    return q.reshape(wl.batch, wl.num_layers, NUM_Q_HEADS, HEAD_DIM).to(torch.float16)


def new_token_kv(m: Materialised, step: int):
    """K and V of the token appended before decode step `step`: [B][L][8][128]
    in the pool's format.  Values N(0, 1); keys get the recent-tail boost
    +k_boost*u (the new token is the most recent position)."""
    wl = m.workload
    device = m.u.device
    gen = torch.Generator(device=device)
    gen.manual_seed(query_seed(wl.seed, step) ^ 0x5A5A5A5A)
    shape = (wl.batch, wl.num_layers, NUM_KV_HEADS, HEAD_DIM)
    k = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    v = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    k += wl.k_boost * m.u[None]
    if wl.kv_format == "e4m3":
        return (k.to(torch.float8_e4m3fn).view(torch.uint8).contiguous(),
                v.to(torch.float8_e4m3fn).view(torch.uint8).contiguous())
    return k.to(torch.float16).contiguous(), v.to(torch.float16).contiguous()
