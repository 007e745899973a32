"""ctypes view of include/kvs.h.  Loading fails loudly when the library is absent."""
from __future__ import annotations

import ctypes
import os

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkvs.so")

KVS_OK = 0
KVS_E_NULL = -1
KVS_E_SHAPE = -2
KVS_E_RANGE = -3
KVS_E_ALIGN = -4
KVS_E_WORKSPACE = -5
KVS_E_POLICY = -6
KVS_E_HIP = -7

KVS_DEV_BAD_BLOCK_ID = 0x1
KVS_DEV_BAD_SEQ_LEN = 0x2
KVS_DEV_BAD_OFFSETS = 0x4
KVS_DEV_STALE_STEP = 0x8
KVS_DEV_POOL_EXHAUSTED = 0x10

KVS_KV_FP16 = 0
KVS_KV_E4M3 = 1
KVS_KV_KIVI2 = 2
KV_FORMATS = {"fp16": KVS_KV_FP16, "e4m3": KVS_KV_E4M3, "kivi2": KVS_KV_KIVI2}

KVS_NEVER_TOUCHED = 0xFFFF_FFFF_FFFF_FFFF
KVS_UNCLASSIFIED = 0xFF
KVS_FLAG_ANCHOR = 0x1

# Every function the header declares, for the export check.
EXPORTS = (
    "kvs_bytes_per_token", "kvs_block_bytes", "kvs_meta_layout", "kvs_decode_split_blocks",
    "kvs_decode_workspace_bytes", "kvs_score_workspace_bytes", "kvs_status_string",
    "kvs_last_error", "kvs_workspace_init", "kvs_device_status", "kvs_decode_step",
    "kvs_meta_init", "kvs_score_update", "kvs_classify", "kvs_set_decode_events",
    "kvs_stream_probe", "kvs_evict_workspace_bytes", "kvs_evict_candidates",
    "kvs_decode_step_e4m3", "kvs_append_workspace_bytes", "kvs_append_kv",
    "kvs_kivi_block_bytes", "kvs_kivi_quantize", "kvs_decode_step_kivi",
    "kvs_kivi_advance_workspace_bytes", "kvs_kivi_advance", "kvs_decode_step_paired",
    "kvs_decode_step_e4m3_paired", "kvs_decode_step_noalloc", "kvs_kivi_quant_len",
)

KVS_NOALLOC_SCRATCH_BYTES = 32 << 20


class Shape(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_tokens", ctypes.c_int32)]


class Policy(ctypes.Structure):
    _fields_ = [("alpha", ctypes.c_double), ("w_recency", ctypes.c_double),
                ("w_ema", ctypes.c_double), ("w_anchor", ctypes.c_double),
                ("t_low", ctypes.c_double), ("t_high", ctypes.c_double)]


# numpy view of kvs_block_meta (64 bytes); offsets checked against the library.
META_DTYPE = np.dtype({
    "names": ["key", "score", "t_touch", "touch_count", "tier", "flags", "reserved0",
              "priority", "reserved1"],
    "formats": [("<u8", (2,)), "<f8", "<u8", "<u4", "u1", "u1", "<u2", "<f8", ("u1", (16,))],
    "offsets": [0, 16, 24, 32, 36, 37, 38, 40, 48],
    "itemsize": 64,
})

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t

_SIGS = {
    "kvs_bytes_per_token": (_sz, [ctypes.POINTER(Shape)]),
    "kvs_block_bytes": (_sz, [ctypes.POINTER(Shape)]),
    "kvs_meta_layout": (_sz, [ctypes.POINTER(ctypes.c_size_t), ctypes.c_int]),
    "kvs_decode_split_blocks": (_i32, [ctypes.POINTER(Shape), _i32, _i32, _i32, _i32, _i32, _i32]),
    "kvs_decode_workspace_bytes": (_sz, [ctypes.POINTER(Shape), _i32, _i32, _i32, _i64, _i32, _i32,
                                         _i32]),
    "kvs_score_workspace_bytes": (_sz, [_i32, _i32]),
    "kvs_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "kvs_last_error": (ctypes.c_char_p, []),
    "kvs_workspace_init": (ctypes.c_int, [_vp, _sz, _vp]),
    "kvs_device_status": (ctypes.c_int, [_vp, _vp, ctypes.POINTER(ctypes.c_uint32)]),
    "kvs_decode_step": (ctypes.c_int, [
        ctypes.POINTER(Shape), _vp, _vp, _i64, _vp, _i32, _vp, _vp, _i32, _i64, _i32, _i32,
        ctypes.c_float, _vp, _vp, ctypes.c_int, _i32, _vp, _sz, _vp]),
    "kvs_decode_step_noalloc": (ctypes.c_int, [
        ctypes.POINTER(Shape), _vp, _vp, _i64, _vp, _i32, _vp, _vp, _i32, _i64, _i32, _i32,
        ctypes.c_float, _vp, _vp, ctypes.c_int, _i32, _vp, _vp]),
    "kvs_decode_step_e4m3": (ctypes.c_int, [
        ctypes.POINTER(Shape), _vp, _vp, _i64, _vp, _i32, _vp, _vp, _i32, _i64, _i32, _i32,
        ctypes.c_float, _vp, _vp, ctypes.c_int, _i32, _vp, _sz, _vp]),
    "kvs_decode_step_paired": (ctypes.c_int, [
        ctypes.POINTER(Shape), _vp, _vp, _i64, _vp, _i32, _vp, _vp, _vp, _i32, _i64, _i32, _i32,
        ctypes.c_float, _vp, _vp, ctypes.c_int, _i32, _vp, _sz, _vp]),
    "kvs_decode_step_e4m3_paired": (ctypes.c_int, [
        ctypes.POINTER(Shape), _vp, _vp, _i64, _vp, _i32, _vp, _vp, _vp, _i32, _i64, _i32, _i32,
        ctypes.c_float, _vp, _vp, ctypes.c_int, _i32, _vp, _sz, _vp]),
    "kvs_decode_step_kivi": (ctypes.c_int, [
        ctypes.POINTER(Shape), _vp, _vp, _i64, _vp, _i64, _vp, _i32, _vp, _vp, _vp, _i32, _i64,
        _i32, _i32, ctypes.c_float, _vp, _vp, ctypes.c_int, _i32, _vp, _sz, _vp]),
    "kvs_kivi_block_bytes": (_sz, [ctypes.POINTER(Shape)]),
    "kvs_kivi_quant_len": (_i32, [_i32, _i32]),
    "kvs_kivi_advance_workspace_bytes": (_sz, [_i32]),
    "kvs_kivi_advance": (ctypes.c_int, [ctypes.POINTER(Shape), _vp, _i64, _vp, _i64, _vp, _i32,
                                        _vp, _vp, _i32, _i32, _vp, _i32, _vp, _vp, _i32, _vp,
                                        _vp, _sz, _vp]),
    "kvs_kivi_quantize": (ctypes.c_int, [ctypes.POINTER(Shape), _vp, _i64, _vp, _i64, _vp, _i32,
                                         _vp, _sz, _vp]),
    "kvs_meta_init": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32, _i64, _i32, _vp]),
    "kvs_score_update": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i64, ctypes.c_uint64,
                                        ctypes.POINTER(Policy), ctypes.c_int, _vp, _sz, _vp]),
    "kvs_classify": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i32, _i64, ctypes.POINTER(Policy),
                                    _vp, _vp]),
    "kvs_set_decode_events": (ctypes.c_int, [_vp, _vp]),
    "kvs_stream_probe": (ctypes.c_int, [_vp, _vp, _sz, ctypes.c_int, _i32, _vp]),
    "kvs_append_workspace_bytes": (_sz, [_i32]),
    "kvs_append_kv": (ctypes.c_int, [ctypes.POINTER(Shape), ctypes.c_int, _vp, _vp, _vp, _i64,
                                     _vp, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _i32,
                                     _i64, _vp, _sz, _vp]),
    "kvs_evict_workspace_bytes": (_sz, [_i32, _i32]),
    "kvs_evict_candidates": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i64, ctypes.c_uint64,
                                            ctypes.c_double, ctypes.c_int, _vp, _vp, _vp, _sz,
                                            _vp]),
}

_LIB = None


class KvsError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code
        self.message = message


def lib() -> ctypes.CDLL:
    """The loaded HIP library.  Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m paged_gqa_kv_amd.build); there is no fallback path")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def check(rc: int) -> None:
    if rc != KVS_OK:
        msg = lib().kvs_last_error().decode(errors="replace")
        raise KvsError(rc, msg or lib().kvs_status_string(rc).decode())
