"""Seeded input recipes for the PBSA workloads.

Workload shapes follow the usage example on the Sparse Forcing project page
("SparseForcingAttention" constructor: total/local/persistent cache sizes, block
size [1,8,8], top-k ratio 0.125) and the benchmark configurations of this
library (tiny fp32 case, the 12-head d=128 decode step, update, backward and an
80-step rollout).  Every array is drawn from numpy's PCG64 with a fixed seed and,
for bf16 workloads, rounded to bfloat16 (round-to-nearest-even) on the CPU so the
oracle and the GPU see bit-identical values.

Salient structure: the abstract reports that attention concentrates on a
persistent subset of salient blocks.  The recipe plants that structure by adding
``alpha * u_h`` (a per-head unit vector) to every key row of a seeded 10% of
the cache blocks.  This is a workload recipe only; nothing here pools, scores,
selects or updates.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# ----------------------------------------------------------------------------
# bf16 helpers (pure bit manipulation of IEEE binary32)
# ----------------------------------------------------------------------------


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, round-to-nearest-even; return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) >> 16
    return u.astype(np.uint16)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); return float32."""
    b = bf16_bits(x).astype(np.uint32) << 16
    return b.view(np.float32)


# ----------------------------------------------------------------------------
# Workload table
# ----------------------------------------------------------------------------

# Keys mirror the C configuration struct.  Sizes are in tokens, as on the
# project page's usage example.
WORKLOADS = {
    # tiny fp32 forward: 16x16 grid (4 blocks of 8x8), 1-frame chunk,
    # 4-frame local ring, 8 persistent blocks, k = 0.25 * 16 = 4.
    "tiny_fp32": dict(
        batch=1, heads=2, head_dim=64, frame_h=16, frame_w=16,
        block_t=1, block_h=8, block_w=8, chunk_frames=1,
        total_cache_size=512 + 1024, local_cache_size=1024,
        persistent_cache_size=512, use_local_block_sparse_attn=1,
        topk_ratio=0.25, softmax_scale=0.0, dtype="fp32",
        seed=0, plant_frac=0.0, alpha=0.0,
    ),
    # the 12-head, d=128 decode step: 30x52 latent grid (1560 tokens, 28
    # blocks per frame with partial edge blocks), 3-frame chunk (4680
    # queries), 9360-token local ring (6 frames, 168 blocks), 168-block /
    # 9360-token persistent cache, top-k ratio 0.125 -> 21 blocks.
    "decode_c1": dict(
        batch=1, heads=12, head_dim=128, frame_h=30, frame_w=52,
        block_t=1, block_h=8, block_w=8, chunk_frames=3,
        total_cache_size=18720, local_cache_size=9360,
        persistent_cache_size=9360, use_local_block_sparse_attn=1,
        topk_ratio=0.125, softmax_scale=0.0, dtype="bf16",
        seed=1, plant_frac=0.1, alpha=4.0,
    ),
}
# the update and backward workloads share the decode step's shape
WORKLOADS["update_c2"] = dict(WORKLOADS["decode_c1"])
WORKLOADS["backward_c3"] = dict(WORKLOADS["decode_c1"], dout_seed=3)
WORKLOADS["rollout_c4"] = dict(WORKLOADS["decode_c1"], seed=4, steps=80,
                               plant_blocks=8, drift_p=0.25, redraw_every=20)
# the decode step with [3,4,4] blocks (the project page's faster block size):
# 104 blocks of 48/24 tokens per 3-frame chunk, 208 local blocks, 208 slots, k = 26
WORKLOADS["decode_344"] = dict(WORKLOADS["decode_c1"], block_t=3, block_h=4, block_w=4, seed=6)


def workload(name: str, **overrides) -> dict:
    w = dict(WORKLOADS[name])
    w.update(overrides)
    return w


# ----------------------------------------------------------------------------
# Shape bookkeeping needed to lay the arrays out (integer only)
# ----------------------------------------------------------------------------


@dataclass(frozen=True)
class _Layout:
    frame_tokens: int
    chunk_tokens: int
    local_tokens: int
    n_slots: int
    slot_cap: int
    cells: tuple          # ((frame0, r0, c0, nt, nh, nw), ...) for the blocks of one chunk
    blocks_per_chunk: int


def _layout(cfg: dict) -> _Layout:
    fh, fw = cfg["frame_h"], cfg["frame_w"]
    bt, bh, bw = cfg["block_t"], cfg["block_h"], cfg["block_w"]
    cf = cfg["chunk_frames"]
    ft = fh * fw
    cells = []
    for f0 in range(0, cf, bt):
        for r0 in range(0, fh, bh):
            for c0 in range(0, fw, bw):
                cells.append((f0, r0, c0, min(bt, cf - f0), min(bh, fh - r0), min(bw, fw - c0)))
    group_tokens = bt * ft
    per_group = len(cells) // max(1, cf // bt)
    n_slots = cfg["persistent_cache_size"] // group_tokens * per_group
    return _Layout(ft, cf * ft, cfg["local_cache_size"], n_slots, bt * bh * bw,
                   tuple(cells), len(cells))


def _cell_tokens(cell, fh, fw) -> np.ndarray:
    f0, r0, c0, nt, nh, nw = cell
    f = np.arange(f0, f0 + nt)[:, None, None]
    r = np.arange(r0, r0 + nh)[None, :, None]
    c = np.arange(c0, c0 + nw)[None, None, :]
    return (f * fh * fw + r * fw + c).reshape(-1)


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def _unit(rng: np.random.Generator, n: int, d: int) -> np.ndarray:
    u = rng.standard_normal(size=(n, d)).astype(np.float64)
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    return u.astype(np.float32)


def _finish(x: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_round(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


# ----------------------------------------------------------------------------
# One decode step's inputs
# ----------------------------------------------------------------------------


def make_step_inputs(cfg: dict, seed: int | None = None) -> dict:
    """Inputs of one decode step.

    Returns float32 arrays (holding bf16 values for bf16 workloads):
      q    [B,H,Nq,D]      query chunk, raster order (frame, row, col)
      k_l  [B,H,NL,D]      local K ring (R chunk slots of Nq tokens), raster
      v_l  [B,H,NL,D]
      k_p  [B,H,S,cap,D]   persistent K slots; rows >= len are zero
      v_p  [B,H,S,cap,D]
    and int32 arrays persist_len [B,H,S], persist_src [B,H,S], ring_head [1].
    Persistent slot s initially holds len = size of chunk block (s mod blocks
    per frame group) random rows and src = -(s+1).
    """
    seed = cfg["seed"] if seed is None else seed
    lay = _layout(cfg)
    B, H, D = cfg["batch"], cfg["heads"], cfg["head_dim"]
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _normal(rng, (B, H, lay.chunk_tokens, D))
    k_l = _normal(rng, (B, H, lay.local_tokens, D))
    v_l = _normal(rng, (B, H, lay.local_tokens, D))
    S, cap = lay.n_slots, lay.slot_cap
    per_group = lay.blocks_per_chunk // max(1, cfg["chunk_frames"] // cfg["block_t"])
    sizes = [c[3] * c[4] * c[5] for c in lay.cells[:per_group]]
    plen = np.array([sizes[s % per_group] for s in range(S)], dtype=np.int32)
    k_p = _normal(rng, (B, H, S, cap, D))
    v_p = _normal(rng, (B, H, S, cap, D))
    rowmask = (np.arange(cap)[None, :] < plen[:, None]).astype(np.float32)
    k_p *= rowmask[None, None, :, :, None]
    v_p *= rowmask[None, None, :, :, None]

    plant_frac = cfg.get("plant_frac", 0.0)
    alpha = cfg.get("alpha", 0.0)
    if plant_frac > 0 and alpha != 0:
        n_local_blocks = lay.local_tokens // lay.chunk_tokens * lay.blocks_per_chunk
        n_cache = S + n_local_blocks
        n_plant = int(round(plant_frac * n_cache))
        u = _unit(rng, B * H, D).reshape(B, H, D)
        fh, fw = cfg["frame_h"], cfg["frame_w"]
        for b in range(B):
            for h in range(H):
                chosen = rng.choice(n_cache, size=n_plant, replace=False)
                for j in np.sort(chosen):
                    if j < S:
                        k_p[b, h, j, : plen[j]] += alpha * u[b, h]
                    else:
                        p = j - S
                        chunk, blk = divmod(p, lay.blocks_per_chunk)
                        tok = chunk * lay.chunk_tokens + _cell_tokens(lay.cells[blk], fh, fw)
                        k_l[b, h, tok] += alpha * u[b, h]

    dt = cfg["dtype"]
    out = dict(
        q=_finish(q, dt), k_l=_finish(k_l, dt), v_l=_finish(v_l, dt),
        k_p=_finish(k_p, dt), v_p=_finish(v_p, dt),
        persist_len=np.broadcast_to(plen, (B, H, S)).astype(np.int32).copy(),
        persist_src=np.broadcast_to(-(np.arange(S, dtype=np.int32) + 1), (B, H, S)).astype(np.int32).copy(),
        ring_head=np.zeros(1, dtype=np.int32),
    )
    return out


def make_dout(cfg: dict, seed: int | None = None) -> np.ndarray:
    """Upstream gradient dO [B,H,Nq,D], i.i.d. N(0,1) (bf16-rounded for bf16 workloads)."""
    seed = cfg.get("dout_seed", 3) if seed is None else seed
    lay = _layout(cfg)
    rng = np.random.Generator(np.random.PCG64(seed))
    x = _normal(rng, (cfg["batch"], cfg["heads"], lay.chunk_tokens, cfg["head_dim"]))
    return _finish(x, cfg["dtype"])


# ----------------------------------------------------------------------------
# Rollout: a stream of chunks with slowly drifting planted blocks
# ----------------------------------------------------------------------------


class RolloutStream:
    """Per-step chunk inputs (q, k_new, v_new) of a long rollout.

    Chunk s (s = -1 is the chunk that already sits in the oldest ring slot at
    step 0) is drawn from its own child seed of ``SeedSequence(seed)``.
    ``plant_blocks`` of the chunk's blocks carry ``alpha * u_h`` on their key
    rows; each planted position moves to a random 4-neighbour within its
    frame's block grid with probability ``drift_p`` per step, and ``u_h`` is
    redrawn every ``redraw_every`` steps.
    """

    def __init__(self, cfg: dict):
        self.cfg = cfg
        self.lay = _layout(cfg)
        B, H = cfg["batch"], cfg["heads"]
        self.steps = cfg.get("steps", 80)
        ss = np.random.SeedSequence(cfg["seed"])
        children = ss.spawn(self.steps + 3)
        self._chunk_seeds = children[: self.steps + 1]
        self._ctrl = np.random.Generator(np.random.PCG64(children[-1]))
        fh, fw = cfg["frame_h"], cfg["frame_w"]
        self.grid = (-(-fh // cfg["block_h"]), -(-fw // cfg["block_w"]))
        nb = self.lay.blocks_per_chunk
        npl = cfg.get("plant_blocks", 8)
        self.pos = np.stack([self._ctrl.choice(nb, size=npl, replace=False) for _ in range(B * H)]).reshape(B, H, npl)
        self.u = _unit(self._ctrl, B * H, cfg["head_dim"]).reshape(B, H, -1)
        self._plans = []
        # precompute the planted positions and directions of every chunk
        for s in range(-1, self.steps):
            if s >= 0 and s % cfg.get("redraw_every", 20) == 0 and s > 0:
                self.u = _unit(self._ctrl, B * H, cfg["head_dim"]).reshape(B, H, -1)
            if s >= 0:
                self._drift()
            self._plans.append((self.pos.copy(), self.u.copy()))

    def _drift(self):
        gr, gc = self.grid
        per_frame = gr * gc
        p = self.cfg.get("drift_p", 0.25)
        moves = ((-1, 0), (1, 0), (0, -1), (0, 1))
        B, H, npl = self.pos.shape
        for b in range(B):
            for h in range(H):
                for i in range(npl):
                    if self._ctrl.random() >= p:
                        continue
                    blk = int(self.pos[b, h, i])
                    f, rc = divmod(blk, per_frame)
                    r, c = divmod(rc, gc)
                    dr, dc = moves[int(self._ctrl.integers(4))]
                    r2, c2 = min(max(r + dr, 0), gr - 1), min(max(c + dc, 0), gc - 1)
                    self.pos[b, h, i] = f * per_frame + r2 * gc + c2

    def chunk(self, s: int) -> dict:
        """Inputs of chunk s in [-1, steps): q [B,H,Nq,D], k, v [B,H,Nq,D]."""
        cfg, lay = self.cfg, self.lay
        B, H, D = cfg["batch"], cfg["heads"], cfg["head_dim"]
        rng = np.random.Generator(np.random.PCG64(self._chunk_seeds[s + 1]))
        q = _normal(rng, (B, H, lay.chunk_tokens, D))
        k = _normal(rng, (B, H, lay.chunk_tokens, D))
        v = _normal(rng, (B, H, lay.chunk_tokens, D))
        pos, u = self._plans[s + 1]
        alpha = cfg.get("alpha", 4.0)
        fh, fw = cfg["frame_h"], cfg["frame_w"]
        for b in range(B):
            for h in range(H):
                for blk in np.unique(pos[b, h]):
                    tok = _cell_tokens(lay.cells[int(blk)], fh, fw)
                    k[b, h, tok] += alpha * u[b, h]
        dt = cfg["dtype"]
        return dict(q=_finish(q, dt), k=_finish(k, dt), v=_finish(v, dt))


def noisy_pass(chunk: dict, cfg: dict, s: int, i: int, n: int) -> dict:
    """Inputs of denoising pass i (0 = noisiest) of n for chunk s: the chunk's
    q, k, v blended with seeded N(0,1) noise, a*x + sqrt(1-a^2)*eps with
    a = (i+1)/(n+1), so every pass keeps unit variance and a fading share of
    the planted structure.  A workload recipe only."""
    a = (i + 1) / (n + 1)
    b = float(np.sqrt(1.0 - a * a))
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg["seed"], 7919, s + 1, i])))
    out = {}
    for name in ("q", "k", "v"):
        x = chunk[name]
        out[name] = _finish(np.float32(a) * x + np.float32(b) * _normal(rng, x.shape), cfg["dtype"])
    return out


def describe(cfg: dict) -> str:
    lay = _layout(cfg)
    return (f"B{cfg['batch']} H{cfg['heads']} d{cfg['head_dim']} {cfg['dtype']} grid {cfg['frame_h']}x{cfg['frame_w']} "
            f"chunk {lay.chunk_tokens} local {lay.local_tokens} slots {lay.n_slots}x{lay.slot_cap}")

