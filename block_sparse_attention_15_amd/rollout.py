"""Chunk-by-chunk PBSA decode loop of one attention layer, graph-capturable.

The training algorithm fragment of Sparse Forcing (review page) runs, for each
generated chunk, the denoising passes with "PBSA with top-K" and then a cache
pass at t = 0 that applies PBSA with top-K and updates the persistent (P) and
local (L) caches.  ``DecodeLoop`` issues exactly those library calls, with
``denoise_passes`` denoising passes per chunk (the pages leave their number
to the model):

* denoising pass i: ``pbsa_ring_append`` of that pass's keys and values into
  the newest ring slot (the slot the last update freed), so the local window
  holds the previous chunk and the current one; then ``pbsa_score_select`` and
  ``pbsa_fwd`` of that pass's queries (no update);
* cache pass: the same with the chunk's t = 0 keys and values, then
  ``pbsa_persist_update``, which evicts the oldest ring chunk into the
  persistent memory and advances ring head and step counter.  With
  ``mass="token"`` the cache pass's forward is ``pbsa_fwd_mass`` and the
  update ranks blocks by their token-exact attention mass instead of the
  pooled mass of score_select.

Every pass has its own staging inputs (q, k, v) and outputs (o, lse, topk),
so one replay of the captured chunk leaves every pass's result readable.
All per-step state (ring head, step counter, slot metadata) lives on the
device, so ``capture()`` records one chunk into a HIP graph (via
``torch.cuda.CUDAGraph``) that is replayed for every chunk after the caller
writes the chunk's inputs into the staging buffers.  Nothing here computes
any part of the method; it only sequences the C ABI calls.
"""
from __future__ import annotations

import torch

from . import api
from .module import PBSACache


class DecodeLoop:
    def __init__(self, plan: api.Plan, cache: PBSACache, device="cuda", mass: str = "pooled",
                 denoise_passes: int = 0):
        if mass not in ("pooled", "token"):
            raise ValueError("mass must be 'pooled' or 'token'")
        if denoise_passes < 0:
            raise ValueError("denoise_passes must be >= 0")
        self.plan = plan
        self.cache = cache
        self.mass_mode = mass
        self.denoise_passes = denoise_passes
        s = api.shapes(plan)
        dt = plan.torch_dtype
        n = denoise_passes + 1          # the last pass is the cache pass (t = 0)

        def z(shape, dtype):
            return [torch.zeros(shape, dtype=dtype, device=device) for _ in range(n)]

        # staging inputs and outputs, one set per pass
        self.qs, self.ks, self.vs = z(s["q"], dt), z(s["q"], dt), z(s["q"], dt)
        self.os, self.lses = z(s["q"], dt), z(s["lse"], torch.float32)
        self.topks = z(s["topk_idx"], torch.int32)
        self.mass = torch.zeros(s["mass"], dtype=torch.float32, device=device)
        self.n_replaced = torch.zeros(s["n_replaced"], dtype=torch.int32, device=device)
        self.ws_score = api.workspace(plan, "score_select", device)
        self.ws_fwd = api.workspace(plan, "fwd", device)
        self.ws_update = api.workspace(plan, "persist_update", device)
        self.ws_fwd_mass = api.workspace(plan, "fwd_mass", device) if mass == "token" else None
        self.graph = None

    # the cache pass's buffers under the names of a single-pass loop
    @property
    def q(self):
        return self.qs[-1]

    @property
    def o(self):
        return self.os[-1]

    @property
    def lse(self):
        return self.lses[-1]

    @property
    def topk(self):
        return self.topks[-1]

    @property
    def kbar_local(self):
        return self.cache.kbar_local

    def load_pass(self, i: int, q, k, v):
        """Copy pass i's q, k, v (device tensors of the chunk shape) into its staging buffers;
        i = denoise_passes (or -1) is the cache pass."""
        self.qs[i].copy_(q)
        self.ks[i].copy_(k)
        self.vs[i].copy_(v)

    def load_chunk(self, q, k, v):
        """Stage the chunk's t = 0 inputs (the cache pass)."""
        self.load_pass(-1, q, k, v)

    def _attend(self, i, stream, token_mass=False):
        c, p = self.cache, self.plan
        api.pbsa_ring_append(p, self.ks[i], self.vs[i], c.ring_head, c.k_local, c.v_local, c.kbar_local, stream)
        api.pbsa_score_select(p, self.qs[i], c.kbar_local, c.ring_head, c.persist_kbar, c.persist_len, self.topks[i],
                              self.mass, self.ws_score, stream)
        if token_mass:
            api.pbsa_fwd_mass(p, self.qs[i], c.k_pers, c.v_pers, c.persist_len, c.k_local, c.v_local,
                              self.topks[i], self.os[i], self.lses[i], self.mass, self.ws_fwd_mass, stream)
        else:
            api.pbsa_fwd(p, self.qs[i], c.k_pers, c.v_pers, c.persist_len, c.k_local, c.v_local, self.topks[i],
                         self.os[i], self.lses[i], self.ws_fwd, stream)

    def denoise_pass(self, i: int, stream=None):
        """Denoising pass i: append its keys/values to the ring, score, select, attend (no update)."""
        if not 0 <= i < self.denoise_passes:
            raise IndexError(f"denoising pass {i} of {self.denoise_passes}")
        self._attend(i, stream)

    def cache_pass(self, stream=None):
        """Append the chunk's t = 0 keys/values, attend, then update the persistent cache."""
        c, p = self.cache, self.plan
        self._attend(-1, stream, token_mass=self.mass_mode == "token")
        api.pbsa_persist_update(p, self.mass, c.k_local, c.v_local, c.kbar_local, c.ring_head, c.step_counter,
                                c.k_pers, c.v_pers, c.persist_len, c.persist_src, c.persist_kbar, self.n_replaced,
                                self.ws_update, stream)

    def step(self, stream=None):
        """One chunk: the denoising passes, then the cache pass."""
        for i in range(self.denoise_passes):
            self.denoise_pass(i, stream)
        self.cache_pass(stream)

    def capture(self) -> torch.cuda.CUDAGraph:
        """Record one ``step`` into a graph.  The library's kernels must have
        run once eagerly before (one-time kernel attribute setup)."""
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                self.step()
        torch.cuda.current_stream().wait_stream(side)
        self.graph = g
        return g

    def replay(self):
        self.graph.replay()
