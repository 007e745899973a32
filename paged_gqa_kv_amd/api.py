"""Thin Python binding of the C ABI (argument marshalling only).

Names follow include/kvs.h without the ``kvs_`` prefix.  Tensor arguments are
torch tensors on the GPU (their data pointers are passed) or plain integers
(raw device addresses); ``stream`` defaults to torch's current stream.  Every
step of the computation runs in the HIP library; nothing here computes.
"""
from __future__ import annotations

import ctypes
import math

import torch

from . import _abi
from ._abi import META_DTYPE, KvsError, Policy, Shape, check, lib  # noqa: F401

DEFAULT_SCALE = 1.0 / math.sqrt(128.0)


def shape(num_layers: int) -> Shape:
    return Shape(num_layers, 64, 8, 128, 16)


def policy(alpha: float, w_recency: float = 0.25, w_ema: float = 0.55, w_anchor: float = 0.20,
           t_low: float = 0.3, t_high: float = 0.6) -> Policy:
    return Policy(alpha, w_recency, w_ema, w_anchor, t_low, t_high)


def _p(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        if not x.is_contiguous():
            raise ValueError("tensors passed to the library must be contiguous "
                             f"(got shape {tuple(x.shape)}, strides {x.stride()})")
        return ctypes.c_void_p(x.data_ptr())
    return ctypes.c_void_p(int(x))


def _s(stream):
    if stream is None:
        if not torch.cuda.is_available():
            return None
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream)) if stream else None


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


# ---- host-only helpers ------------------------------------------------------

def bytes_per_token(shp: Shape) -> int:
    return lib().kvs_bytes_per_token(ctypes.byref(shp))


def block_bytes(shp: Shape) -> int:
    return lib().kvs_block_bytes(ctypes.byref(shp))


def meta_layout():
    offs = (ctypes.c_size_t * 9)()
    size = lib().kvs_meta_layout(offs, 9)
    return size, list(offs)


def _fmt(kv_format) -> int:
    return _abi.KV_FORMATS[kv_format] if isinstance(kv_format, str) else int(kv_format)


def decode_split_blocks(shp: Shape, batch: int, max_blocks: int, layer_begin: int,
                        layer_end: int, split_blocks: int = 0, kv_format="fp16") -> int:
    return lib().kvs_decode_split_blocks(ctypes.byref(shp), _fmt(kv_format), batch, max_blocks,
                                         layer_begin, layer_end, split_blocks)


def decode_workspace_bytes(shp: Shape, batch: int, max_blocks: int, total_blocks: int,
                           layer_begin: int, layer_end: int, split_blocks: int = 0,
                           kv_format="fp16") -> int:
    return lib().kvs_decode_workspace_bytes(ctypes.byref(shp), _fmt(kv_format), batch,
                                            max_blocks, total_blocks, layer_begin, layer_end,
                                            split_blocks)


KIVI_RESIDUAL_TOKENS = 128   # the fp16 window of the newest ~128 tokens


def kivi_quant_len(seq_len: int, residual_tokens: int = KIVI_RESIDUAL_TOKENS) -> int:
    """The library's window rule (kvs_kivi_quant_len): quantised tokens of a
    seq_len-token sequence."""
    v = lib().kvs_kivi_quant_len(int(seq_len), int(residual_tokens))
    if v < 0:
        raise ValueError(f"invalid seq_len {seq_len} or residual_tokens {residual_tokens}")
    return v


def kivi_block_bytes(shp: Shape) -> int:
    return lib().kvs_kivi_block_bytes(ctypes.byref(shp))


def score_workspace_bytes(batch: int, max_blocks: int) -> int:
    return lib().kvs_score_workspace_bytes(batch, max_blocks)


def status_string(code: int) -> str:
    return lib().kvs_status_string(code).decode()


def last_error() -> str:
    return lib().kvs_last_error().decode()


# ---- device entry points ----------------------------------------------------

def set_decode_events(before, after) -> None:
    """Raw hipEvent_t handles (ints) recorded around the decode kernel, or None, None."""
    check(lib().kvs_set_decode_events(_p(before), _p(after)))


PROBE_DEFAULT_GRID = 2048   # work-groups kvs_stream_probe launches for grid 0


def stream_probe(src, dst, nbytes: int, mode: int, grid: int = 0, stream=None) -> None:
    """kvs_stream_probe.  Where src / dst are tensors their sizes are checked
    first: src must hold nbytes; dst nbytes (copy) or one 32-bit word per lane,
    grid x 256 words (read)."""
    if hasattr(src, "numel") and _nbytes(src) < nbytes:
        raise ValueError(f"src holds {_nbytes(src)} bytes, the probe reads {nbytes}")
    if hasattr(dst, "numel"):
        need = nbytes if mode == 1 else (grid if grid > 0 else PROBE_DEFAULT_GRID) * 256 * 4
        if _nbytes(dst) < need:
            raise ValueError(f"dst holds {_nbytes(dst)} bytes, mode {mode} at grid {grid} "
                             f"writes {need}")
    check(lib().kvs_stream_probe(_p(src), _p(dst), nbytes, mode, grid, _s(stream)))


def workspace_init(workspace, nbytes=None, stream=None) -> None:
    n = _nbytes(workspace) if nbytes is None else nbytes
    check(lib().kvs_workspace_init(_p(workspace), n, _s(stream)))


def device_status(workspace, stream=None) -> int:
    bits = ctypes.c_uint32(0)
    check(lib().kvs_device_status(_p(workspace), _s(stream), ctypes.byref(bits)))
    return bits.value


def decode_step(shp: Shape, q, kv_pool, pool_blocks: int, block_table, max_blocks: int,
                seq_lens, meta_offsets, batch: int, total_blocks: int, layer_begin: int,
                layer_end: int, scale: float, out, block_mass, accumulate: int,
                split_blocks: int, workspace, workspace_bytes=None, stream=None) -> None:
    ws_bytes = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    check(lib().kvs_decode_step(ctypes.byref(shp), _p(q), _p(kv_pool), pool_blocks,
                                _p(block_table), max_blocks, _p(seq_lens), _p(meta_offsets),
                                batch, total_blocks, layer_begin, layer_end, scale, _p(out),
                                _p(block_mass), accumulate, split_blocks, _p(workspace),
                                ws_bytes, _s(stream)))


def decode_step_noalloc(shp: Shape, q, kv_pool, pool_blocks: int, block_table, max_blocks: int,
                        seq_lens, meta_offsets, batch: int, total_blocks: int, layer_begin: int,
                        layer_end: int, scale: float, out, block_mass, accumulate: int,
                        split_blocks: int, status, stream=None) -> None:
    """kvs_decode_step_noalloc: the decode step with the library's own scratch;
    `status` is a caller-owned device uint32 word for the sticky status bits."""
    check(lib().kvs_decode_step_noalloc(ctypes.byref(shp), _p(q), _p(kv_pool), pool_blocks,
                                        _p(block_table), max_blocks, _p(seq_lens),
                                        _p(meta_offsets), batch, total_blocks, layer_begin,
                                        layer_end, scale, _p(out), _p(block_mass), accumulate,
                                        split_blocks, _p(status), _s(stream)))


def decode_step_e4m3(shp: Shape, q, kv_pool, pool_blocks: int, block_table, max_blocks: int,
                     seq_lens, meta_offsets, batch: int, total_blocks: int, layer_begin: int,
                     layer_end: int, scale: float, out, block_mass, accumulate: int,
                     split_blocks: int, workspace, workspace_bytes=None, stream=None) -> None:
    ws_bytes = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    check(lib().kvs_decode_step_e4m3(ctypes.byref(shp), _p(q), _p(kv_pool), pool_blocks,
                                     _p(block_table), max_blocks, _p(seq_lens), _p(meta_offsets),
                                     batch, total_blocks, layer_begin, layer_end, scale, _p(out),
                                     _p(block_mass), accumulate, split_blocks, _p(workspace),
                                     ws_bytes, _s(stream)))


def decode_step_paired(shp: Shape, q, kv_pool, pool_blocks: int, block_table, max_blocks: int,
                       seq_lens, pair_role, meta_offsets, batch: int, total_blocks: int,
                       layer_begin: int, layer_end: int, scale: float, out, block_mass,
                       accumulate: int, split_blocks: int, workspace, workspace_bytes=None,
                       stream=None) -> None:
    ws_bytes = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    check(lib().kvs_decode_step_paired(ctypes.byref(shp), _p(q), _p(kv_pool), pool_blocks,
                                       _p(block_table), max_blocks, _p(seq_lens), _p(pair_role),
                                       _p(meta_offsets), batch, total_blocks, layer_begin,
                                       layer_end, scale, _p(out), _p(block_mass), accumulate,
                                       split_blocks, _p(workspace), ws_bytes, _s(stream)))


def decode_step_e4m3_paired(shp: Shape, q, kv_pool, pool_blocks: int, block_table,
                            max_blocks: int, seq_lens, pair_role, meta_offsets, batch: int,
                            total_blocks: int, layer_begin: int, layer_end: int, scale: float,
                            out, block_mass, accumulate: int, split_blocks: int, workspace,
                            workspace_bytes=None, stream=None) -> None:
    ws_bytes = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    check(lib().kvs_decode_step_e4m3_paired(ctypes.byref(shp), _p(q), _p(kv_pool), pool_blocks,
                                            _p(block_table), max_blocks, _p(seq_lens),
                                            _p(pair_role), _p(meta_offsets), batch, total_blocks,
                                            layer_begin, layer_end, scale, _p(out),
                                            _p(block_mass), accumulate, split_blocks,
                                            _p(workspace), ws_bytes, _s(stream)))


def decode_step_kivi(shp: Shape, q, kv_pool, pool_blocks: int, kivi_pool, kivi_blocks: int,
                     block_table, max_blocks: int, seq_lens, quant_lens, meta_offsets, batch: int,
                     total_blocks: int, layer_begin: int, layer_end: int, scale: float, out,
                     block_mass, accumulate: int, split_blocks: int, workspace,
                     workspace_bytes=None, stream=None) -> None:
    ws_bytes = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    check(lib().kvs_decode_step_kivi(ctypes.byref(shp), _p(q), _p(kv_pool), pool_blocks,
                                     _p(kivi_pool), kivi_blocks, _p(block_table), max_blocks,
                                     _p(seq_lens), _p(quant_lens), _p(meta_offsets), batch,
                                     total_blocks, layer_begin, layer_end, scale, _p(out),
                                     _p(block_mass), accumulate, split_blocks, _p(workspace),
                                     ws_bytes, _s(stream)))


def kivi_quantize(shp: Shape, kv_pool, pool_blocks: int, kivi_pool, kivi_blocks: int, pairs,
                  n_pairs: int, workspace, workspace_bytes=None, stream=None) -> None:
    ws_bytes = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    check(lib().kvs_kivi_quantize(ctypes.byref(shp), _p(kv_pool), pool_blocks, _p(kivi_pool),
                                  kivi_blocks, _p(pairs), n_pairs, _p(workspace), ws_bytes,
                                  _s(stream)))


def kivi_advance_workspace_bytes(batch: int) -> int:
    return lib().kvs_kivi_advance_workspace_bytes(batch)


def kivi_advance(shp: Shape, kv_pool, pool_blocks: int, kivi_pool, kivi_blocks: int, block_table,
                 max_blocks: int, seq_lens, quant_lens, batch: int, residual_tokens: int,
                 kivi_free, kivi_free_capacity: int, kivi_free_top, fp16_free,
                 fp16_free_capacity: int, fp16_free_top, workspace, workspace_bytes=None,
                 stream=None) -> None:
    ws_bytes = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    check(lib().kvs_kivi_advance(ctypes.byref(shp), _p(kv_pool), pool_blocks, _p(kivi_pool),
                                 kivi_blocks, _p(block_table), max_blocks, _p(seq_lens),
                                 _p(quant_lens), batch, residual_tokens, _p(kivi_free),
                                 kivi_free_capacity, _p(kivi_free_top), _p(fp16_free),
                                 fp16_free_capacity, _p(fp16_free_top), _p(workspace), ws_bytes,
                                 _s(stream)))


def meta_init(meta, meta_offsets, seq_ids, batch: int, max_blocks: int, total_blocks: int,
              anchor_blocks: int = 1, stream=None) -> None:
    check(lib().kvs_meta_init(_p(meta), _p(meta_offsets), _p(seq_ids), batch, max_blocks,
                              total_blocks, anchor_blocks, _s(stream)))


def score_update(meta, block_mass, meta_offsets, seq_lens, batch: int, max_blocks: int,
                 total_blocks: int, step: int, pol: Policy, classify: int, workspace,
                 workspace_bytes=None, stream=None) -> None:
    ws_bytes = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    check(lib().kvs_score_update(_p(meta), _p(block_mass), _p(meta_offsets), _p(seq_lens), batch,
                                 max_blocks, total_blocks, step, ctypes.byref(pol), classify,
                                 _p(workspace), ws_bytes, _s(stream)))


def classify(meta, meta_offsets, seq_lens, batch: int, max_blocks: int, total_blocks: int,
             pol: Policy, tiers_out=None, stream=None) -> None:
    check(lib().kvs_classify(_p(meta), _p(meta_offsets), _p(seq_lens), batch, max_blocks,
                             total_blocks, ctypes.byref(pol), _p(tiers_out), _s(stream)))


def append_workspace_bytes(batch: int) -> int:
    return lib().kvs_append_workspace_bytes(batch)


def append_kv(shp: Shape, kv_elem_bytes: int, k_new, v_new, kv_pool, pool_blocks: int,
              block_table, max_blocks: int, seq_lens, free_stack, free_capacity: int, free_top,
              meta, meta_offsets, seq_ids, anchor_blocks: int, batch: int, total_blocks: int,
              workspace, workspace_bytes=None, stream=None) -> None:
    ws_bytes = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    check(lib().kvs_append_kv(ctypes.byref(shp), kv_elem_bytes, _p(k_new), _p(v_new),
                              _p(kv_pool), pool_blocks, _p(block_table), max_blocks,
                              _p(seq_lens), _p(free_stack), free_capacity, _p(free_top), _p(meta),
                              _p(meta_offsets), _p(seq_ids), anchor_blocks, batch, total_blocks,
                              _p(workspace), ws_bytes, _s(stream)))


def evict_workspace_bytes(batch: int, max_blocks: int) -> int:
    return lib().kvs_evict_workspace_bytes(batch, max_blocks)


def evict_candidates(meta, meta_offsets, seq_lens, active, batch: int, max_blocks: int,
                     total_blocks: int, now: int, alpha: float, exclude_pinned: int, out_block,
                     out_key, workspace, workspace_bytes=None, stream=None) -> None:
    ws_bytes = _nbytes(workspace) if workspace_bytes is None else workspace_bytes
    check(lib().kvs_evict_candidates(_p(meta), _p(meta_offsets), _p(seq_lens), _p(active),
                                     batch, max_blocks,
                                     total_blocks, now, alpha, exclude_pinned, _p(out_block),
                                     _p(out_key), _p(workspace), ws_bytes, _s(stream)))


def records(meta: torch.Tensor):
    """Copy a device record array (uint8 [n][64] or any 64-byte-row tensor) to a
    numpy structured array with META_DTYPE."""
    raw = meta.detach().contiguous().view(torch.uint8).cpu().numpy()
    return raw.view(META_DTYPE).reshape(-1)
