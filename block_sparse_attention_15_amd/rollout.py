"""Chunk-by-chunk PBSA decode loop of one attention layer, graph-capturable.

The training algorithm fragment of Sparse Forcing (review page) runs, for each
generated chunk, the denoising passes with "PBSA with top-K" and then a cache
pass at t = 0 that applies PBSA with top-K and updates the persistent (P) and
local (L) caches.  ``DecodeLoop`` issues exactly those library calls:

* ``denoise_pass()``: score_select + fwd on the current chunk (no update);
* ``cache_pass()``:   ring_append of the chunk's K/V into the free ring slot,
  score_select, fwd, persist_update (which advances ring head and step).
  With ``mass="token"`` the forward of the cache pass is ``pbsa_fwd_mass``
  and the update ranks blocks by their token-exact attention mass instead of
  the pooled mass of score_select.

All per-step state (ring head, step counter, slot metadata) lives on the
device, so ``capture()`` records one step into a HIP graph (via
``torch.cuda.CUDAGraph``) that can be replayed for every chunk after the
caller copies the chunk's q / k / v into the staging buffers.  Nothing here
computes any part of the method; it only sequences the C ABI calls.
"""
from __future__ import annotations

import torch

from . import api
from .module import PBSACache


class DecodeLoop:
    def __init__(self, plan: api.Plan, cache: PBSACache, device="cuda", mass: str = "pooled"):
        if mass not in ("pooled", "token"):
            raise ValueError("mass must be 'pooled' or 'token'")
        self.plan = plan
        self.cache = cache
        self.mass_mode = mass
        s = api.shapes(plan)
        dt = plan.torch_dtype
        self.q = torch.zeros(s["q"], dtype=dt, device=device)       # staging: current chunk queries
        self.k_new = torch.zeros(s["q"], dtype=dt, device=device)   # staging: current chunk keys
        self.v_new = torch.zeros(s["q"], dtype=dt, device=device)   # staging: current chunk values
        self.o = torch.zeros(s["q"], dtype=dt, device=device)
        self.lse = torch.zeros(s["lse"], dtype=torch.float32, device=device)
        self.topk = torch.zeros(s["topk_idx"], dtype=torch.int32, device=device)
        self.mass = torch.zeros(s["mass"], dtype=torch.float32, device=device)
        self.kbar_local = torch.zeros(s["kbar_local"], dtype=torch.float32, device=device)
        self.n_replaced = torch.zeros(s["n_replaced"], dtype=torch.int32, device=device)
        self.ws_score = api.workspace(plan, "score_select", device)
        self.ws_fwd = api.workspace(plan, "fwd", device)
        self.ws_update = api.workspace(plan, "persist_update", device)
        self.ws_fwd_mass = api.workspace(plan, "fwd_mass", device) if mass == "token" else None
        self.graph = None

    def load_chunk(self, q, k, v):
        """Copy one chunk's q, k, v (device tensors of the chunk shape) into the staging buffers."""
        self.q.copy_(q)
        self.k_new.copy_(k)
        self.v_new.copy_(v)

    def _attend(self, stream=None):
        c, p = self.cache, self.plan
        api.pbsa_score_select(p, self.q, c.k_local, c.ring_head, c.persist_kbar, c.persist_len, self.topk,
                              self.mass, self.kbar_local, self.ws_score, stream)
        api.pbsa_fwd(p, self.q, c.k_pers, c.v_pers, c.persist_len, c.k_local, c.v_local, self.topk, self.o,
                     self.lse, self.ws_fwd, stream)

    def denoise_pass(self, stream=None):
        """score_select + fwd of the current chunk against the caches (no update)."""
        self._attend(stream)

    def cache_pass(self, stream=None):
        """Append the chunk's K/V to the ring, attend, then update the persistent cache."""
        c, p = self.cache, self.plan
        api.pbsa_ring_append(p, self.k_new, self.v_new, c.ring_head, c.k_local, c.v_local, stream)
        if self.mass_mode == "token":
            api.pbsa_score_select(p, self.q, c.k_local, c.ring_head, c.persist_kbar, c.persist_len, self.topk,
                                  self.mass, self.kbar_local, self.ws_score, stream)
            api.pbsa_fwd_mass(p, self.q, c.k_pers, c.v_pers, c.persist_len, c.k_local, c.v_local, self.topk, self.o,
                              self.lse, self.mass, self.ws_fwd_mass, stream)
        else:
            self._attend(stream)
        api.pbsa_persist_update(p, self.mass, c.k_local, c.v_local, self.kbar_local, c.ring_head, c.step_counter,
                                c.k_pers, c.v_pers, c.persist_len, c.persist_src, c.persist_kbar, self.n_replaced,
                                self.ws_update, stream)

    def step(self, denoise_passes: int = 0, stream=None):
        """One chunk: ``denoise_passes`` denoising passes, then the cache pass."""
        for _ in range(denoise_passes):
            self.denoise_pass(stream)
        self.cache_pass(stream)

    def capture(self, denoise_passes: int = 0) -> torch.cuda.CUDAGraph:
        """Record one ``step`` into a graph.  The library's kernels must have
        run once eagerly before (one-time kernel attribute setup)."""
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                self.step(denoise_passes)
        torch.cuda.current_stream().wait_stream(side)
        self.graph = g
        return g

    def replay(self):
        self.graph.replay()
