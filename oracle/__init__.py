"""fp64 CPU oracle for the paged GQA decode step and per-block scoring.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this
package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may call it.  It shares no code,
constants generator or helper with the HIP library; its inputs are the
materialised tensors of ``workload`` (copied to host), and its outputs are
compared element by element with the library's.

Sources (cited by page title and section throughout):

* "KV-Cache Offloading for LLM Inference -- Visual Reference" (v6.0):
  Sec. 2 (attention), Sec. 3 Diagram 3.1 (KV size), Sec. 11 Diagrams
  11.1-11.2 (EMA), Sec. 12 Diagrams 12.1-12.2 (priority, tier cut points).
* "GQA Per-Head Scoring Streams": query heads 8g..8g+7 read KV head g;
  640 (layer, KV-head) streams aggregated into one score per
  (sequence, block); the 64-byte per-block state.
* "KV cache offload" architecture post, "Top row": block table of physical
  ids, paged placement.
* "Fitting a Million Tokens", Sec. 01: KV bytes per token.

Parity status of each function is stated in its module.
"""
from . import arithmetic, attention, scoring  # noqa: F401
