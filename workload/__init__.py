"""Seeded synthetic inputs for the paged GQA decode + block-scoring path.

This package holds no arithmetic of the method itself: it only draws the
query, the paged K/V pool and the block tables.  Both the oracle tests and
the HIP path consume what it produces.
"""
from .recipe import (  # noqa: F401
    HEAD_DIM,
    NUM_KV_HEADS,
    NUM_Q_HEADS,
    BLOCK_TOKENS,
    Workload,
    Materialised,
    WORKLOADS,
    as_e4m3,
    as_kivi2,
    kivi_placement,
    custom,
    materialise,
    make_query,
    new_token_kv,
    query_seed,
)
