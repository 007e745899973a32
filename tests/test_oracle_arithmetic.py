"""Oracle byte accounting pinned to the figures the pages print."""
import json
import math
import os

from oracle import arithmetic as A

GOLD = os.path.join(os.path.dirname(__file__), "golden", "arithmetic.json")


def _gold():
    with open(GOLD) as f:
        return json.load(f)


def _round_like(x, printed: str) -> str:
    decimals = len(printed.split(".")[1]) if "." in printed else 0
    return f"{x:.{decimals}f}"


def test_printed_figures():
    g = _gold()
    m = g["model"]
    shape = (m["layers"], m["kv_heads"], m["head_dim"], m["elem_bytes"])
    per_tok = A.kv_bytes_per_token(*shape)
    blk = A.block_bytes(*shape, m["block_tokens"])
    for row in g["printed"]:
        what, unit, val = row["what"], row["unit"], row["value"]
        if what == "KV bytes per token":
            assert per_tok == val
            assert per_tok == 320 * 1024
        elif what == "one 16-token block":
            assert _round_like(blk / 2**20, val) == val
            assert blk == 16 * per_tok == 5 * 2**20
        elif what.startswith("context"):
            b = A.context_bytes(row["tokens"], *shape)
            scale = {"GiB": 2**30, "GB": 1e9}[unit]
            assert _round_like(b / scale, val) == val, (row, b)
        elif what == "blocks at 128K":
            assert row["tokens"] // m["block_tokens"] == val
        elif what == "metadata at 128K":
            assert A.metadata_bytes(row["blocks"]) == val == 512 * 1024
        elif what == "metadata overhead at 128K":
            kv = A.context_bytes(row["blocks"] * m["block_tokens"], *shape)
            pct = 100.0 * A.metadata_bytes(row["blocks"]) / kv
            assert _round_like(pct, val) == val
            # the same ratio as one 64-byte record against one block
            assert math.isclose(pct, 100.0 * 64 / blk)
        else:  # pragma: no cover
            raise AssertionError(f"unhandled golden row {what}")


def test_exact_integers():
    # 128K context is exactly 40 GiB; 8K is exactly 2.5 GiB.
    assert A.context_bytes(131072, 80, 8, 128, 2) == 42_949_672_960 == 40 * 2**30
    assert A.context_bytes(8192, 80, 8, 128, 2) == 2_684_354_560
    # one 16-token block of one layer (all 8 KV heads, K and V) is 64 KiB;
    # one (layer, K-or-V, KV-head) tile is 4 KiB.
    assert A.block_bytes(1, 8, 128, 2, 16) == 64 * 1024
    assert A.block_bytes(1, 1, 128, 2, 16) // 2 == 4096


def test_block_move_times():
    g = _gold()
    blk = A.block_bytes(80, 8, 128, 2, 16)
    for case in g["block_move_us"]["cases"]:
        us = blk / (case["gb_per_s"] * 1e9) * 1e6
        assert _round_like(us, case["printed_us"]) == case["printed_us"]
