"""``SparseForcingAttention``: the module interface of the Sparse Forcing
project page's usage example, on top of the C ABI.

The page constructs the module with the cache sizes, the block size and the
top-k ratio, and calls it as ``attn(query, key_persistent, value_persistent,
key_local, value_local)``.  Here the persistent cache carries its per-slot
metadata (valid length, source id, pooled key) in a ``PBSACache``; calling
with ``update=True`` runs the cache pass of the paper's algorithm (attention,
then the persistent update and the ring advance).
"""
from __future__ import annotations

import torch

from . import api


class PBSACache:
    """Device state of one layer's KV caches (persistent slots + local ring)."""

    def __init__(self, plan: api.Plan, device="cuda"):
        s = api.shapes(plan)
        dt = plan.torch_dtype
        self.plan = plan
        self.k_pers = torch.zeros(s["k_pers"], dtype=dt, device=device)
        self.v_pers = torch.zeros(s["k_pers"], dtype=dt, device=device)
        self.persist_len = torch.zeros(s["persist_len"], dtype=torch.int32, device=device)
        self.persist_src = torch.full(s["persist_len"], -(2 ** 31), dtype=torch.int32, device=device)
        self.persist_kbar = torch.zeros(s["persist_kbar"], dtype=torch.float32, device=device)
        self.k_local = torch.zeros(s["k_local"], dtype=dt, device=device)
        self.v_local = torch.zeros(s["k_local"], dtype=dt, device=device)
        self.kbar_local = torch.zeros(s["kbar_local"], dtype=torch.float32, device=device)  # ring metadata
        self.ring_head = torch.zeros(1, dtype=torch.int32, device=device)
        self.step_counter = torch.zeros(1, dtype=torch.int32, device=device)

    STATE = ("k_pers", "v_pers", "persist_len", "persist_src", "persist_kbar", "k_local", "v_local", "kbar_local",
             "ring_head", "step_counter")

    def refresh_pooled_keys(self, stream=None):
        """Recompute the pooled keys of the persistent slots and of the local
        ring (after their keys were written from outside the library)."""
        api.pbsa_pool_slots(self.plan, self.k_pers, self.persist_len, self.persist_kbar, stream)
        api.pbsa_pool_local(self.plan, self.k_local, self.kbar_local, stream)

    def state_dict(self) -> dict:
        """Host copies of every tensor of the cache state (a checkpoint).
        Waits for the work queued on the current stream."""
        torch.cuda.current_stream().synchronize()
        return {k: getattr(self, k).detach().to("cpu", copy=True) for k in self.STATE}

    def load_state_dict(self, state: dict):
        """Restore a checkpoint taken by ``state_dict`` (same plan)."""
        for k in self.STATE:
            t = getattr(self, k)
            src = state[k]
            if tuple(src.shape) != tuple(t.shape) or src.dtype != t.dtype:
                raise ValueError(f"{k}: checkpoint has {tuple(src.shape)} {src.dtype}, cache has "
                                 f"{tuple(t.shape)} {t.dtype}")
            t.copy_(src)


class SparseForcingAttention:
    def __init__(self, total_cache_size: int, local_cache_size: int, persistent_cache_size: int,
                 kv_cache_mode: str = "sparse_forcing", sparse_kv_block_size=(1, 8, 8), max_seq_len: int = 32760,
                 use_local_block_sparse_attn: bool = True, local_block_sparse_topk_ratio: float = 0.125, *,
                 batch: int = 1, heads: int = 12, head_dim: int = 128, frame_h: int = 30, frame_w: int = 52,
                 chunk_frames: int = 3, softmax_scale: float = 0.0, dtype: str = "bf16", sink_slots: int = 0,
                 mass: str = "pooled", device="cuda"):
        if kv_cache_mode != "sparse_forcing":
            raise ValueError("only kv_cache_mode='sparse_forcing' is implemented")
        bt, bh, bw = sparse_kv_block_size
        self.max_seq_len = max_seq_len
        self.plan = api.pbsa_plan(dict(
            batch=batch, heads=heads, head_dim=head_dim, frame_h=frame_h, frame_w=frame_w,
            block_t=bt, block_h=bh, block_w=bw, chunk_frames=chunk_frames,
            total_cache_size=total_cache_size, local_cache_size=local_cache_size,
            persistent_cache_size=persistent_cache_size,
            use_local_block_sparse_attn=int(bool(use_local_block_sparse_attn)),
            topk_ratio=local_block_sparse_topk_ratio, softmax_scale=softmax_scale, dtype=dtype,
            sink_slots=sink_slots))
        if mass not in ("pooled", "token"):
            raise ValueError("mass must be 'pooled' or 'token'")
        self.mass_mode = mass
        p, s = self.plan, api.shapes(self.plan)
        self.device = device
        self.ws_score = api.workspace(p, "score_select", device)
        self.ws_bwd = None
        self.ws_update = api.workspace(p, "persist_update", device)
        self.ws_fwd = api.workspace(p, "fwd", device)
        self.ws_fwd_mass = api.workspace(p, "fwd_mass", device) if mass == "token" else None
        self.topk_idx = torch.empty(s["topk_idx"], dtype=torch.int32, device=device)
        self.mass = torch.empty(s["mass"], dtype=torch.float32, device=device)
        self.n_replaced = torch.empty(s["n_replaced"], dtype=torch.int32, device=device)

    def new_cache(self) -> PBSACache:
        return PBSACache(self.plan, self.device)

    def __call__(self, query, key_persistent=None, value_persistent=None, key_local=None, value_local=None, *,
                 cache: PBSACache | None = None, update: bool = False, stream=None):
        """Attention of ``query`` over the persistent and selected local blocks.

        With ``cache`` the caches and their metadata come from it, and
        ``key_local`` / ``value_local`` are the current chunk's keys and values
        (the shape of ``query``): they are written into the newest slot of the
        cache's local ring first, so the chunk attends its own keys.  With
        ``update=True`` the call is the cache pass: after attention the
        persistent cache is updated from the oldest ring chunk and the ring
        advances.  Without ``cache``, the four key/value tensors are the caches
        themselves, and every persistent slot is treated as full (its pooled
        keys are computed on the fly).
        """
        p = self.plan
        if cache is not None:
            if key_persistent is not None or value_persistent is not None:
                raise ValueError("with a cache, the persistent keys and values come from it")
            if (key_local is None) != (value_local is None):
                raise ValueError("key_local and value_local go together")
            if key_local is not None:
                api.pbsa_ring_append(p, key_local, value_local, cache.ring_head, cache.k_local, cache.v_local,
                                     cache.kbar_local, stream)
        else:
            if update:
                raise ValueError("update=True needs a cache (the persistent state it updates)")
            cache = PBSACache.__new__(PBSACache)
            cache.plan = p
            cache.k_pers, cache.v_pers = key_persistent, value_persistent
            cache.k_local, cache.v_local = key_local, value_local
            shp = api.shapes(p)
            cache.persist_len = torch.full(shp["persist_len"], p.slot_rows, dtype=torch.int32, device=query.device)
            cache.persist_src = torch.arange(shp["persist_len"][-1], dtype=torch.int32,
                                             device=query.device).expand(shp["persist_len"]).contiguous()
            cache.persist_kbar = torch.empty(shp["persist_kbar"], dtype=torch.float32, device=query.device)
            cache.kbar_local = torch.empty(shp["kbar_local"], dtype=torch.float32, device=query.device)
            cache.ring_head = torch.zeros(1, dtype=torch.int32, device=query.device)
            cache.step_counter = torch.zeros(1, dtype=torch.int32, device=query.device)
            cache.refresh_pooled_keys(stream)
        o = torch.empty_like(query)
        lse = torch.empty(api.shapes(p)["lse"], dtype=torch.float32, device=query.device)
        api.pbsa_score_select(p, query, cache.kbar_local, cache.ring_head, cache.persist_kbar, cache.persist_len,
                              self.topk_idx, self.mass, self.ws_score, stream)
        if update and self.mass_mode == "token":
            api.pbsa_fwd_mass(p, query, cache.k_pers, cache.v_pers, cache.persist_len, cache.k_local, cache.v_local,
                              self.topk_idx, o, lse, self.mass, self.ws_fwd_mass, stream)
        else:
            api.pbsa_fwd(p, query, cache.k_pers, cache.v_pers, cache.persist_len, cache.k_local, cache.v_local,
                         self.topk_idx, o, lse, self.ws_fwd, stream)
        if update:
            api.pbsa_persist_update(p, self.mass, cache.k_local, cache.v_local, cache.kbar_local, cache.ring_head,
                                    cache.step_counter, cache.k_pers, cache.v_pers, cache.persist_len,
                                    cache.persist_src, cache.persist_kbar, self.n_replaced, self.ws_update, stream)
        self.last_lse = lse
        return o
