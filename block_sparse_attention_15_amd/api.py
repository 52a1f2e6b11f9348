"""Python binding of the PBSA C ABI: same names as include/pbsa.h.

Each function checks shapes, dtypes and devices of its torch tensors (so no
kernel can be handed a buffer that is too small), then passes raw pointers to
the C library on the current HIP stream.  All arithmetic happens in the HIP
kernels; nothing here computes any part of the method.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib

_CONFIG_KEYS = ("batch", "heads", "head_dim", "frame_h", "frame_w", "block_t", "block_h", "block_w",
                "chunk_frames", "total_cache_size", "local_cache_size", "persistent_cache_size",
                "use_local_block_sparse_attn", "topk_ratio", "softmax_scale")


class PbsaError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with {_lib.STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


@dataclass
class Plan:
    cfg: _lib.PbsaConfig
    blocks_per_chunk: int
    local_blocks: int
    ring_chunks: int
    persistent_slots: int
    slot_rows: int
    topk: int
    chunk_tokens: int
    max_block_tokens: int
    ws_score_select: int
    ws_fwd: int
    ws_bwd: int
    ws_persist_update: int
    ws_fwd_mass: int

    @property
    def B(self):
        return self.cfg.batch

    @property
    def H(self):
        return self.cfg.heads

    @property
    def D(self):
        return self.cfg.head_dim

    @property
    def local_tokens(self):
        return self.cfg.local_cache_size

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.cfg.dtype == _lib.PBSA_BF16 else torch.float32


def make_config(d: dict) -> _lib.PbsaConfig:
    c = _lib.PbsaConfig()
    for k in _CONFIG_KEYS:
        setattr(c, k, d[k])
    c.sink_slots = int(d.get("sink_slots", 0))
    c.bwd_ds_max_mb = int(d.get("bwd_ds_max_mb", 0))
    dt = d.get("dtype", "bf16")
    c.dtype = {"bf16": _lib.PBSA_BF16, "fp32": _lib.PBSA_FP32}[dt] if isinstance(dt, str) else int(dt)
    return c


def _call(name: str, *args):
    lib = _lib.load()
    st = getattr(lib, name)(*args)
    if st != _lib.PBSA_OK:
        raise PbsaError(name, st, lib.pbsa_last_error().decode())


def pbsa_plan(cfg) -> Plan:
    c = cfg if isinstance(cfg, _lib.PbsaConfig) else make_config(cfg)
    info = _lib.PbsaPlanInfo()
    _call("pbsa_plan", ctypes.byref(c), ctypes.byref(info))
    return Plan(c, *(getattr(info, f) for f, _ in _lib.PbsaPlanInfo._fields_))


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t: torch.Tensor | None, shape, dtype, name: str):
    if t is None:
        if shape is None:
            return None
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _ws(ws: torch.Tensor | None, need: int):
    if need == 0 and ws is None:
        return None, 0
    if ws is None:
        raise ValueError("workspace required")
    if not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    return ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size()


def shapes(p: Plan) -> dict:
    B, H, D = p.B, p.H, p.D
    S, C, nq, nl = p.persistent_slots, p.slot_rows, p.blocks_per_chunk, p.local_blocks
    return dict(q=(B, H, p.chunk_tokens, D), k_local=(B, H, p.local_tokens, D),
                k_pers=(B, H, S, C, D), persist_len=(B, H, S), persist_kbar=(B, H, S, D),
                topk_idx=(B, H, nq, p.topk), mass=(B, H, S + nl), kbar_local=(B, H, nl, D),
                lse=(B, H, p.chunk_tokens), n_replaced=(B, H), ring_head=(1,))


def workspace(p: Plan, which: str, device="cuda") -> torch.Tensor | None:
    n = getattr(p, "ws_" + which)
    if n == 0:
        return None
    return torch.empty(n, dtype=torch.uint8, device=device)


def pbsa_pool_slots(p: Plan, k_pers, persist_len, persist_kbar, stream=None):
    s = shapes(p)
    _call("pbsa_pool_slots", ctypes.byref(p.cfg), _ptr(k_pers, s["k_pers"], p.torch_dtype, "k_pers"),
          _ptr(persist_len, s["persist_len"], torch.int32, "persist_len"),
          _ptr(persist_kbar, s["persist_kbar"], torch.float32, "persist_kbar"), _stream(stream))


def pbsa_pool_local(p: Plan, k_local, kbar_local, stream=None):
    """Pooled keys of every local block of the ring (for a ring written from outside the library)."""
    s = shapes(p)
    _call("pbsa_pool_local", ctypes.byref(p.cfg), _ptr(k_local, s["k_local"], p.torch_dtype, "k_local"),
          _ptr(kbar_local, s["kbar_local"], torch.float32, "kbar_local"), _stream(stream))


def pbsa_score_select(p: Plan, q, kbar_local, ring_head, persist_kbar, persist_len, topk_idx, mass, ws, stream=None):
    s = shapes(p)
    w, nb = _ws(ws, p.ws_score_select)
    _call("pbsa_score_select", ctypes.byref(p.cfg), _ptr(q, s["q"], p.torch_dtype, "q"),
          _ptr(kbar_local, s["kbar_local"], torch.float32, "kbar_local"),
          _ptr(ring_head, s["ring_head"], torch.int32, "ring_head"),
          _ptr(persist_kbar, s["persist_kbar"], torch.float32, "persist_kbar"),
          _ptr(persist_len, s["persist_len"], torch.int32, "persist_len"),
          _ptr(topk_idx, s["topk_idx"], torch.int32, "topk_idx"),
          _ptr(mass, s["mass"], torch.float32, "mass"), w, nb, _stream(stream))


def pbsa_score_select_noalloc(p: Plan, q, kbar_local, ring_head, persist_kbar, persist_len, topk_idx, mass,
                              stream=None):
    """pbsa_score_select with the library's static scratch instead of a workspace (allocates nothing)."""
    s = shapes(p)
    _call("pbsa_score_select_noalloc", ctypes.byref(p.cfg), _ptr(q, s["q"], p.torch_dtype, "q"),
          _ptr(kbar_local, s["kbar_local"], torch.float32, "kbar_local"),
          _ptr(ring_head, s["ring_head"], torch.int32, "ring_head"),
          _ptr(persist_kbar, s["persist_kbar"], torch.float32, "persist_kbar"),
          _ptr(persist_len, s["persist_len"], torch.int32, "persist_len"),
          _ptr(topk_idx, s["topk_idx"], torch.int32, "topk_idx"),
          _ptr(mass, s["mass"], torch.float32, "mass"), _stream(stream))


def pbsa_fwd(p: Plan, q, k_pers, v_pers, persist_len, k_local, v_local, topk_idx, o, lse, ws=None, stream=None):
    s = shapes(p)
    dt = p.torch_dtype
    w, nb = _ws(ws, p.ws_fwd)
    _call("pbsa_fwd", ctypes.byref(p.cfg), _ptr(q, s["q"], dt, "q"), _ptr(k_pers, s["k_pers"], dt, "k_pers"),
          _ptr(v_pers, s["k_pers"], dt, "v_pers"), _ptr(persist_len, s["persist_len"], torch.int32, "persist_len"),
          _ptr(k_local, s["k_local"], dt, "k_local"), _ptr(v_local, s["k_local"], dt, "v_local"),
          _ptr(topk_idx, s["topk_idx"], torch.int32, "topk_idx"), _ptr(o, s["q"], dt, "o"),
          _ptr(lse, s["lse"], torch.float32, "lse"), w, nb, _stream(stream))


def pbsa_fwd_mass(p: Plan, q, k_pers, v_pers, persist_len, k_local, v_local, topk_idx, o, lse, mass, ws,
                  stream=None):
    """pbsa_fwd plus the token-exact mass of every candidate block into ``mass``."""
    s = shapes(p)
    dt = p.torch_dtype
    w, nb = _ws(ws, p.ws_fwd_mass)
    _call("pbsa_fwd_mass", ctypes.byref(p.cfg), _ptr(q, s["q"], dt, "q"), _ptr(k_pers, s["k_pers"], dt, "k_pers"),
          _ptr(v_pers, s["k_pers"], dt, "v_pers"), _ptr(persist_len, s["persist_len"], torch.int32, "persist_len"),
          _ptr(k_local, s["k_local"], dt, "k_local"), _ptr(v_local, s["k_local"], dt, "v_local"),
          _ptr(topk_idx, s["topk_idx"], torch.int32, "topk_idx"), _ptr(o, s["q"], dt, "o"),
          _ptr(lse, s["lse"], torch.float32, "lse"), _ptr(mass, s["mass"], torch.float32, "mass"), w, nb,
          _stream(stream))


def pbsa_bwd(p: Plan, q, k_pers, v_pers, persist_len, k_local, v_local, topk_idx, o, lse, dout,
             dq, dk_pers, dv_pers, dk_local, dv_local, ws, stream=None):
    s = shapes(p)
    dt = p.torch_dtype
    f32 = torch.float32
    w, nb = _ws(ws, p.ws_bwd)
    _call("pbsa_bwd", ctypes.byref(p.cfg), _ptr(q, s["q"], dt, "q"), _ptr(k_pers, s["k_pers"], dt, "k_pers"),
          _ptr(v_pers, s["k_pers"], dt, "v_pers"), _ptr(persist_len, s["persist_len"], torch.int32, "persist_len"),
          _ptr(k_local, s["k_local"], dt, "k_local"), _ptr(v_local, s["k_local"], dt, "v_local"),
          _ptr(topk_idx, s["topk_idx"], torch.int32, "topk_idx"), _ptr(o, s["q"], dt, "o"),
          _ptr(lse, s["lse"], f32, "lse"), _ptr(dout, s["q"], dt, "dout"), _ptr(dq, s["q"], f32, "dq"),
          _ptr(dk_pers, s["k_pers"], f32, "dk_pers"), _ptr(dv_pers, s["k_pers"], f32, "dv_pers"),
          _ptr(dk_local, s["k_local"], f32, "dk_local"), _ptr(dv_local, s["k_local"], f32, "dv_local"),
          w, nb, _stream(stream))


def pbsa_persist_update(p: Plan, mass, k_local, v_local, kbar_local, ring_head, step_counter, k_pers, v_pers,
                        persist_len, persist_src, persist_kbar, n_replaced, ws, stream=None):
    """``ring_head`` and ``step_counter`` are int32 device tensors of shape (1,),
    both advanced by the call (the step id tags the admitted blocks' src)."""
    s = shapes(p)
    dt = p.torch_dtype
    w, nb = _ws(ws, p.ws_persist_update)
    _call("pbsa_persist_update", ctypes.byref(p.cfg), _ptr(mass, s["mass"], torch.float32, "mass"),
          _ptr(k_local, s["k_local"], dt, "k_local"), _ptr(v_local, s["k_local"], dt, "v_local"),
          _ptr(kbar_local, s["kbar_local"], torch.float32, "kbar_local"),
          _ptr(ring_head, s["ring_head"], torch.int32, "ring_head"),
          _ptr(step_counter, s["ring_head"], torch.int32, "step_counter"),
          _ptr(k_pers, s["k_pers"], dt, "k_pers"), _ptr(v_pers, s["k_pers"], dt, "v_pers"),
          _ptr(persist_len, s["persist_len"], torch.int32, "persist_len"),
          _ptr(persist_src, s["persist_len"], torch.int32, "persist_src"),
          _ptr(persist_kbar, s["persist_kbar"], torch.float32, "persist_kbar"),
          _ptr(n_replaced, s["n_replaced"], torch.int32, "n_replaced"), w, nb, _stream(stream))


def pbsa_ring_append(p: Plan, k_new, v_new, ring_head, k_local, v_local, kbar_local, stream=None):
    """Write a chunk's keys/values into the newest ring slot and pool its keys into ``kbar_local``."""
    s = shapes(p)
    dt = p.torch_dtype
    _call("pbsa_ring_append", ctypes.byref(p.cfg), _ptr(k_new, s["q"], dt, "k_new"), _ptr(v_new, s["q"], dt, "v_new"),
          _ptr(ring_head, s["ring_head"], torch.int32, "ring_head"), _ptr(k_local, s["k_local"], dt, "k_local"),
          _ptr(v_local, s["k_local"], dt, "v_local"), _ptr(kbar_local, s["kbar_local"], torch.float32, "kbar_local"),
          _stream(stream))


def pbsa_device_status(out, clear: bool = True, stream=None):
    """Copy the device's sticky status bits into ``out`` (int32 device tensor
    of shape (1,)), resetting them when ``clear``; see PBSA_DEVICE_* in _lib."""
    _call("pbsa_device_status", _ptr(out, (1,), torch.int32, "out"), ctypes.c_int32(1 if clear else 0),
          _stream(stream))
