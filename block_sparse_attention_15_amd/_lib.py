"""ctypes view of the C ABI declared in include/pbsa.h (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpbsa.so")

PBSA_OK = 0
PBSA_ERR_INVALID_ARG = -1
PBSA_ERR_UNSUPPORTED = -2
PBSA_ERR_ALIGNMENT = -3
PBSA_ERR_WORKSPACE = -4
PBSA_ERR_HIP = -5
PBSA_BF16 = 0
PBSA_FP32 = 1
PBSA_DEVICE_BAD_RING_HEAD = 1
PBSA_DEVICE_BAD_STEP_COUNTER = 2

STATUS_NAMES = {0: "PBSA_OK", -1: "PBSA_ERR_INVALID_ARG", -2: "PBSA_ERR_UNSUPPORTED",
                -3: "PBSA_ERR_ALIGNMENT", -4: "PBSA_ERR_WORKSPACE", -5: "PBSA_ERR_HIP"}


class PbsaConfig(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("frame_h", ctypes.c_int32), ("frame_w", ctypes.c_int32),
        ("block_t", ctypes.c_int32), ("block_h", ctypes.c_int32), ("block_w", ctypes.c_int32),
        ("chunk_frames", ctypes.c_int32),
        ("total_cache_size", ctypes.c_int64), ("local_cache_size", ctypes.c_int64),
        ("persistent_cache_size", ctypes.c_int64),
        ("use_local_block_sparse_attn", ctypes.c_int32),
        ("topk_ratio", ctypes.c_float), ("softmax_scale", ctypes.c_float),
        ("dtype", ctypes.c_int32), ("sink_slots", ctypes.c_int32), ("bwd_ds_max_mb", ctypes.c_int32),
    ]


class PbsaPlanInfo(ctypes.Structure):
    _fields_ = [
        ("blocks_per_chunk", ctypes.c_int32), ("local_blocks", ctypes.c_int32),
        ("ring_chunks", ctypes.c_int32), ("persistent_slots", ctypes.c_int32),
        ("slot_rows", ctypes.c_int32), ("topk", ctypes.c_int32),
        ("chunk_tokens", ctypes.c_int32), ("max_block_tokens", ctypes.c_int32),
        ("ws_score_select", ctypes.c_size_t), ("ws_fwd", ctypes.c_size_t),
        ("ws_bwd", ctypes.c_size_t), ("ws_persist_update", ctypes.c_size_t),
        ("ws_fwd_mass", ctypes.c_size_t),
    ]


_P = ctypes.c_void_p
_CFG = ctypes.POINTER(PbsaConfig)
SIGNATURES = {
    "pbsa_plan": [_CFG, ctypes.POINTER(PbsaPlanInfo)],
    "pbsa_pool_slots": [_CFG, _P, _P, _P, _P],
    "pbsa_pool_local": [_CFG, _P, _P, _P],
    "pbsa_score_select": [_CFG, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "pbsa_score_select_noalloc": [_CFG, _P, _P, _P, _P, _P, _P, _P, _P],
    "pbsa_fwd": [_CFG, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "pbsa_fwd_mass": [_CFG, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "pbsa_bwd": [_CFG] + [_P] * 15 + [_P, ctypes.c_size_t, _P],
    "pbsa_persist_update": [_CFG, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "pbsa_ring_append": [_CFG, _P, _P, _P, _P, _P, _P, _P],
    "pbsa_device_status": [_P, ctypes.c_int32, _P],
}

_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libpbsa.so; raise ImportError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(f"{path} not found: build it with `python -m block_sparse_attention_15_amd.build`")
    lib = ctypes.CDLL(path)
    for name, args in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.pbsa_last_error.argtypes = []
    lib.pbsa_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def exported_symbols() -> list:
    return list(SIGNATURES) + ["pbsa_last_error"]
