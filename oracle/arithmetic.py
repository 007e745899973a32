"""Byte accounting of the paged KV cache (exact integer arithmetic).

Pinned by the figures the pages print (tests/golden/arithmetic.json).
"""


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """One token keeps a key and a value vector per layer per KV head.

    Visual Reference Sec. 3, Diagram 3.1 (size = L x H_kv x seq x d x 2 x
    bytes); Fitting a Million Tokens Sec. 01 (the same product).
    """
    return 2 * layers * kv_heads * head_dim * elem_bytes


def block_bytes(layers: int, kv_heads: int, head_dim: int, elem_bytes: int,
                block_tokens: int) -> int:
    """A block is block_tokens tokens of every layer and KV head, moved as one
    unit (GQA Per-Head Scoring Streams, the 16-token, 5.00 MiB block)."""
    return block_tokens * kv_bytes_per_token(layers, kv_heads, head_dim, elem_bytes)


def context_bytes(tokens: int, layers: int, kv_heads: int, head_dim: int,
                  elem_bytes: int) -> int:
    """KV of one sequence of `tokens` positions (Visual Reference Sec. 10,
    the 2.50 GiB / 40.0 GiB figures)."""
    return tokens * kv_bytes_per_token(layers, kv_heads, head_dim, elem_bytes)


def metadata_bytes(n_blocks: int, record_bytes: int = 64) -> int:
    """Per-block state is one fixed-size record per block (GQA Per-Head Scoring
    Streams, "Per-block state (64 bytes)")."""
    return n_blocks * record_bytes
