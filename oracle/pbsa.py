"""Plain, slow, CPU definition of one PBSA decode step (test infrastructure only).

Sources (titles of the pages this follows):
  * "Sparse Forcing: Native Trainable Sparse Attention for Real-time
    Autoregressive Diffusion Video Generation" -- abstract: attention over a
    persistent set of salient blocks plus a dynamically selected local
    neighbourhood inside a sliding window; a kernel (PBSA) that does the sparse
    attention and the memory update.
  * Project page "Sparse Forcing", feature list (local block-sparse attention
    with persistent blocks, learned top-k selection, full gradient support) and
    its usage example (``SparseForcingAttention(total_cache_size=18720,
    local_cache_size=9360, persistent_cache_size=9360,
    sparse_kv_block_size=[1,8,8], local_block_sparse_topk_ratio=0.125, ...)``
    called as ``attn(query, key_persistent, value_persistent, key_local,
    value_local)``).
  * Review page, fragment of the paper's training algorithm: the t=0 cache
    pass applies PBSA with top-K and updates the persistent (P) and local (L)
    caches; the denoising passes apply PBSA with top-K only.

Everything the pages leave open is fixed by an explicit reading (``READINGS``).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

EMPTY_SRC = np.int32(-(2 ** 31))

READINGS = {
    "R1": "block score = softmax_scale * mean-pooled q . mean-pooled k; pools divide by the valid token count",
    "R2": "selection is per (batch, head, query block); query blocks use the same tiling as key blocks",
    "R3": "top-k candidates are all local blocks, current chunk included; no causal mask inside the chunk",
    "R4": "k = clamp(ceil(ratio * n_local_blocks - 1e-6), 1, n_local_blocks); ratio 1 when sparse attention is off",
    "R5": "exact score ties go to the lower logical local index (oldest chunk first); ids returned are physical, ascending",
    "R6": "partial edge blocks keep their true size (24..64 tokens); invalid rows never enter pooling, softmax or gradients",
    "R7": "persistent slots = persistent_cache_size / (block_t * frame_tokens) * blocks per frame group; slot capacity block_t*block_h*block_w rows",
    "R8": "persistent and selected local keys share one softmax",
    "R9": "the update runs once per chunk step, after the forward, on that step's queries",
    "R10": "the evicted blocks are those of the oldest local ring chunk",
    "R11": "block mass = sum over query blocks of a softmax (over valid persistent slots and all local blocks) of pooled scores",
    "R12": "keep the top S of (valid persistent slots + evicted blocks) by mass; ties: incumbents first, then lower index",
    "R13": "vacated slots (ascending) receive admitted entrants (ascending); unused slots are emptied; padding rows are zero",
    "R14": "persistent pooled keys are carried as slot metadata, copied from the entrant's pooled key",
    "R15": "near-tie: boundary gap < 1e-4 * (max - min) of the row's (or head's) oracle scores",
    "R16": "inputs are bf16-rounded (or fp32); attention and gradients in float64; decisions in float32",
    "R17": "gradients flow to q, k_p, v_p, k_l, v_l only; the block mask is fixed",
    "R20": "sink pattern (project page feature list): the first sink_slots persistent slots are pinned: never "
           "candidates for eviction; an empty sink slot j takes block j of the chunk leaving the local window, so "
           "a rollout that starts from an empty persistent cache pins the first frame's blocks",
    "R21": "per generated chunk, the caller's number of denoising passes (score, select and attend only) and "
           "then the cache pass (attend, then update); each pass first writes its own keys and values into the "
           "newest local ring slot, so every pass attends the current chunk",
    "R19": "token-exact mass (the other reading of R11, chosen by the caller): block mass = sum over the chunk's "
           "query tokens of the probability their PBSA softmax puts on the block's rows; 0 for empty slots and for "
           "local blocks no query block selected",
}


# ----------------------------------------------------------------------------
# Geometry  (project page usage example: block size [1,8,8], cache sizes)
# ----------------------------------------------------------------------------


@dataclass
class Geometry:
    B: int
    H: int
    D: int
    frame_h: int
    frame_w: int
    bt: int
    bh: int
    bw: int
    chunk_frames: int
    frame_tokens: int
    chunk_tokens: int
    n_qblk: int          # blocks per chunk (= query blocks)
    R: int               # local ring chunk slots
    n_lblk: int          # local blocks
    S: int               # persistent slots
    cap: int             # rows per persistent slot
    topk: int
    scale: float
    block_tok: list      # per chunk block: token offsets inside the chunk (raster order)
    block_len: np.ndarray
    n_sink: int = 0      # pinned leading persistent slots (reading R20)

    def local_tokens_of(self, p: int) -> np.ndarray:
        c, blk = divmod(p, self.n_qblk)
        return c * self.chunk_tokens + self.block_tok[blk]

    def logical_of(self, p: int, ring_head: int) -> int:
        c, blk = divmod(p, self.n_qblk)
        return ((c - ring_head) % self.R) * self.n_qblk + blk


def geometry(cfg: dict) -> Geometry:
    """Derived sizes of a configuration (readings R4, R6, R7).

    A frame of frame_h x frame_w tokens is cut into ceil(h/8) x ceil(w/8)
    blocks in block-row-major order; block (r, c) covers rows [8r, min(8r+8,h))
    and columns [8c, min(8c+8,w)); its tokens are listed in raster order.
    With block_t > 1 a block spans block_t consecutive frames.
    """
    fh, fw = cfg["frame_h"], cfg["frame_w"]
    bt, bh, bw = cfg["block_t"], cfg["block_h"], cfg["block_w"]
    cf = cfg["chunk_frames"]
    if cfg["total_cache_size"] != cfg["local_cache_size"] + cfg["persistent_cache_size"]:
        raise ValueError("total_cache_size must equal local + persistent")
    if cf % bt:
        raise ValueError("chunk_frames must be a multiple of block_t")
    ft = fh * fw
    ct = cf * ft
    if cfg["local_cache_size"] % ct:
        raise ValueError("local cache must hold whole chunks")
    if cfg["persistent_cache_size"] % (bt * ft):
        raise ValueError("persistent cache must hold whole frame groups")
    block_tok = []
    for f0 in range(0, cf, bt):
        for r0 in range(0, fh, bh):
            for c0 in range(0, fw, bw):
                f = np.arange(f0, f0 + bt)[:, None, None]
                r = np.arange(r0, min(r0 + bh, fh))[None, :, None]
                c = np.arange(c0, min(c0 + bw, fw))[None, None, :]
                block_tok.append((f * ft + r * fw + c).reshape(-1))
    n_qblk = len(block_tok)
    per_group = n_qblk // (cf // bt)
    R = cfg["local_cache_size"] // ct
    n_lblk = R * n_qblk
    S = cfg["persistent_cache_size"] // (bt * ft) * per_group
    if cfg.get("use_local_block_sparse_attn", 1):
        k = math.ceil(float(cfg["topk_ratio"]) * n_lblk - 1e-6)
        k = min(max(k, 1), n_lblk)
    else:
        k = n_lblk
    scale = cfg.get("softmax_scale", 0.0) or 1.0 / math.sqrt(cfg["head_dim"])
    n_sink = int(cfg.get("sink_slots", 0))
    if not 0 <= n_sink <= min(S, n_qblk):
        raise ValueError("sink_slots must be in [0, min(persistent slots, blocks per chunk)]")
    return Geometry(cfg["batch"], cfg["heads"], cfg["head_dim"], fh, fw, bt, bh, bw, cf, ft, ct,
                    n_qblk, R, n_lblk, S, bt * bh * bw, k, float(scale), block_tok,
                    np.array([len(t) for t in block_tok], dtype=np.int32), n_sink)


# ----------------------------------------------------------------------------
# Pooling (reading R1: mean over the block's valid tokens)
# ----------------------------------------------------------------------------


def pool_query_blocks(q: np.ndarray, g: Geometry) -> np.ndarray:
    """qbar[b,h,j] = mean of q over the tokens of chunk block j; float32 result."""
    out = np.empty((g.B, g.H, g.n_qblk, g.D), dtype=np.float64)
    q64 = q.astype(np.float64)
    for j, tok in enumerate(g.block_tok):
        out[:, :, j] = q64[:, :, tok].mean(axis=2)
    return out.astype(np.float32)


def pool_local_blocks(k_l: np.ndarray, g: Geometry) -> np.ndarray:
    """kbar_l[b,h,p] = mean of local keys over physical local block p; float32."""
    out = np.empty((g.B, g.H, g.n_lblk, g.D), dtype=np.float64)
    k64 = k_l.astype(np.float64)
    for p in range(g.n_lblk):
        out[:, :, p] = k64[:, :, g.local_tokens_of(p)].mean(axis=2)
    return out.astype(np.float32)


def pool_slots(k_p: np.ndarray, plen: np.ndarray) -> np.ndarray:
    """kbar_p[b,h,s] = mean of the first len rows of slot s (zero for empty slots); float32."""
    B, H, S, cap, D = k_p.shape
    out = np.zeros((B, H, S, D), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for s in range(S):
                n = int(plen[b, h, s])
                if n > 0:
                    out[b, h, s] = k_p[b, h, s, :n].astype(np.float64).mean(axis=0)
    return out.astype(np.float32)


# ----------------------------------------------------------------------------
# Scoring and top-k selection (project page: "learned top-k selection";
# abstract: "dynamically selected local neighborhood"; readings R1-R5)
# ----------------------------------------------------------------------------


def block_scores(qbar: np.ndarray, kbar: np.ndarray, scale: float) -> np.ndarray:
    """s[b,h,i,j] = scale * (qbar[b,h,i] . kbar[b,h,j]) in float32."""
    s = np.matmul(qbar.astype(np.float32), np.swapaxes(kbar.astype(np.float32), -1, -2))
    return (s * np.float32(scale)).astype(np.float32)


def select_topk(scores: np.ndarray, g: Geometry, ring_head: int) -> np.ndarray:
    """Top-k local blocks per (b, h, query block).

    scores[b,h,i,p] are indexed by physical local block p.  Blocks are ranked by
    descending score, exact ties by ascending logical index (R5); the k winners
    are returned as physical ids in ascending order.
    """
    logical = np.array([g.logical_of(p, ring_head) for p in range(g.n_lblk)])
    out = np.empty(scores.shape[:3] + (g.topk,), dtype=np.int32)
    for b in range(g.B):
        for h in range(g.H):
            for i in range(g.n_qblk):
                order = np.lexsort((logical, -scores[b, h, i].astype(np.float64)))
                out[b, h, i] = np.sort(order[: g.topk])
    return out


def pooled_mass(qbar: np.ndarray, kbar_p: np.ndarray, plen: np.ndarray, kbar_l: np.ndarray,
                g: Geometry) -> np.ndarray:
    """Pooled attention mass per candidate block (reading R11), float32.

    For each query block i, a softmax over the pooled logits
    scale * qbar_i . kbar_j, j running over valid persistent slots and all local
    blocks; mass_j = sum over query blocks i.  Output [B,H,S+n_lblk]: slot s at
    index s (0 for empty slots), physical local block p at index S+p.
    """
    out = np.zeros((g.B, g.H, g.S + g.n_lblk), dtype=np.float32)
    for b in range(g.B):
        for h in range(g.H):
            valid = np.nonzero(plen[b, h] > 0)[0]
            keys = np.concatenate([kbar_p[b, h, valid], kbar_l[b, h]], axis=0)
            lg = block_scores(qbar[b, h], keys, g.scale)                  # [n_qblk, nv + n_lblk]
            m = lg.max(axis=1, keepdims=True)
            e = np.exp((lg - m).astype(np.float32)).astype(np.float32)
            p = (e / e.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)
            col = p.sum(axis=0, dtype=np.float32)
            out[b, h, valid] = col[: len(valid)]
            out[b, h, g.S:] = col[len(valid):]
    return out


def score_select(q, k_l, ring_head: int, kbar_p, plen, g: Geometry) -> dict:
    """Pool, score, select and compute masses for one decode step."""
    qbar = pool_query_blocks(q, g)
    kbar_l = pool_local_blocks(k_l, g)
    scores = block_scores(qbar, kbar_l, g.scale)
    return dict(qbar=qbar, kbar_l=kbar_l, scores=scores,
                topk_idx=select_topk(scores, g, ring_head),
                mass=pooled_mass(qbar, kbar_p, plen, kbar_l, g))


# ----------------------------------------------------------------------------
# Attention (abstract; project page "local block-sparse attention with
# persistent blocks"; readings R3, R6, R8)
# ----------------------------------------------------------------------------


def _key_rows(k_p, v_p, plen, k_l, v_l, sel, b, h, g):
    """Keys and values a query block attends: valid persistent rows, then selected local blocks."""
    ks, vs, where = [], [], []
    for s in range(g.S):
        n = int(plen[b, h, s])
        if n:
            ks.append(k_p[b, h, s, :n])
            vs.append(v_p[b, h, s, :n])
            where.append(("p", s, n))
    for p in sel:
        tok = g.local_tokens_of(int(p))
        ks.append(k_l[b, h, tok])
        vs.append(v_l[b, h, tok])
        where.append(("l", int(p), tok))
    return (np.concatenate(ks).astype(np.float64), np.concatenate(vs).astype(np.float64), where)


def attend(q, k_p, v_p, plen, k_l, v_l, topk_idx, g: Geometry, qblocks=None):
    """O and LSE (natural log) of PBSA in float64.

    Every query token of chunk block i attends all valid rows of all
    persistent slots plus every token of its selected local blocks, with a
    single softmax over that union (R8).  ``qblocks`` restricts the work to a
    subset of query blocks; other rows are NaN.
    """
    Nq = g.chunk_tokens
    O = np.full((g.B, g.H, Nq, g.D), np.nan)
    L = np.full((g.B, g.H, Nq), np.nan)
    blocks = range(g.n_qblk) if qblocks is None else qblocks
    for b in range(g.B):
        for h in range(g.H):
            for i in blocks:
                K, V, _ = _key_rows(k_p, v_p, plen, k_l, v_l, topk_idx[b, h, i], b, h, g)
                tok = g.block_tok[i]
                Q = q[b, h, tok].astype(np.float64)
                S = g.scale * (Q @ K.T)
                m = S.max(axis=1, keepdims=True)
                P = np.exp(S - m)
                l = P.sum(axis=1, keepdims=True)
                O[b, h, tok] = (P @ V) / l
                L[b, h, tok] = (m + np.log(l))[:, 0]
    return O, L


def token_mass(q, k_p, plen, k_l, topk_idx, g: Geometry) -> np.ndarray:
    """Token-exact attention mass per candidate block (reading R19).

    For every query token t of query block i, P_t is the softmax of
    scale * q_t . k over t's PBSA key set (valid persistent rows plus the
    rows of block i's selected local blocks, as in ``attend``); the mass of a
    block is the sum over all query tokens of the probability P_t puts on
    that block's rows.  Accumulated in float64 and returned as float32 (the
    precision in which the update ranks masses), in the layout of
    ``pooled_mass``: slot s at index s, physical local block p at S+p.
    """
    out = np.zeros((g.B, g.H, g.S + g.n_lblk))
    for b in range(g.B):
        for h in range(g.H):
            for i in range(g.n_qblk):
                K, _, where = _key_rows(k_p, k_p, plen, k_l, k_l, topk_idx[b, h, i], b, h, g)
                Q = q[b, h, g.block_tok[i]].astype(np.float64)
                S = g.scale * (Q @ K.T)
                P = np.exp(S - S.max(axis=1, keepdims=True))
                P /= P.sum(axis=1, keepdims=True)
                col = P.sum(axis=0)                       # probability received by each key row
                r = 0
                for kind, idx, ext in where:
                    n = ext if kind == "p" else len(ext)
                    out[b, h, idx if kind == "p" else g.S + idx] += col[r:r + n].sum()
                    r += n
    return out.astype(np.float32)


def attend_bwd(q, k_p, v_p, plen, k_l, v_l, topk_idx, dout, g: Geometry, qblocks=None):
    """Gradients of sum(dout * O) w.r.t. q, k_p, v_p, k_l, v_l (float64), fixed mask (R17).

    Standard softmax-attention calculus on each query block's key set:
    P = softmax(scale Q K^T), dV = P^T dO, dP = dO V^T, D = rowsum(dO * O),
    dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q.  Padding rows and
    unselected blocks get zero gradient.  ``qblocks`` restricts the sum to
    those query blocks: their dQ rows are exact, other dQ rows stay zero and
    dK / dV hold only those blocks' contributions.
    """
    dq = np.zeros((g.B, g.H, g.chunk_tokens, g.D))
    dk_p = np.zeros(k_p.shape)
    dv_p = np.zeros(v_p.shape)
    dk_l = np.zeros(k_l.shape)
    dv_l = np.zeros(v_l.shape)
    blocks = range(g.n_qblk) if qblocks is None else qblocks
    for b in range(g.B):
        for h in range(g.H):
            for i in blocks:
                K, V, where = _key_rows(k_p, v_p, plen, k_l, v_l, topk_idx[b, h, i], b, h, g)
                tok = g.block_tok[i]
                Q = q[b, h, tok].astype(np.float64)
                dO = dout[b, h, tok].astype(np.float64)
                S = g.scale * (Q @ K.T)
                P = np.exp(S - S.max(axis=1, keepdims=True))
                P /= P.sum(axis=1, keepdims=True)
                O = P @ V
                dV = P.T @ dO
                dP = dO @ V.T
                Dr = (dO * O).sum(axis=1, keepdims=True)
                dS = P * (dP - Dr)
                dq[b, h, tok] = g.scale * (dS @ K)
                dK = g.scale * (dS.T @ Q)
                r = 0
                for kind, idx, ext in where:
                    if kind == "p":
                        dk_p[b, h, idx, :ext] += dK[r:r + ext]
                        dv_p[b, h, idx, :ext] += dV[r:r + ext]
                        r += ext
                    else:
                        n = len(ext)
                        dk_l[b, h, ext] += dK[r:r + n]
                        dv_l[b, h, ext] += dV[r:r + n]
                        r += n
    return dict(dq=dq, dk_p=dk_p, dv_p=dv_p, dk_l=dk_l, dv_l=dv_l)


# ----------------------------------------------------------------------------
# Persistent-cache update (abstract: "compress, preserve, and update these
# persistent blocks"; algorithm fragment: "Update P and L" in the cache pass;
# readings R9-R14)
# ----------------------------------------------------------------------------


def update_decisions(mass, plen, ring_head: int, g: Geometry):
    """Which incumbents stay and which evicted blocks enter, per (b, h).

    Candidates: valid persistent slots (mass[s]) and the n_qblk blocks e of the
    oldest ring chunk (mass[S + phys(e)]).  Rank by descending mass; ties put
    incumbents before entrants, then the lower slot / block index.  The first
    min(S, #candidates) are kept.  Returns keep[B,H,S] (bool) and
    admit[B,H,n_qblk] (bool).

    Sink slots (reading R20), s < n_sink, are not candidates: a valid one is
    always kept, an empty one always admits evicted block e = s; the other
    candidates compete for the remaining S - n_sink places.
    """
    keep = np.zeros((g.B, g.H, g.S), dtype=bool)
    admit = np.zeros((g.B, g.H, g.n_qblk), dtype=bool)
    old = ring_head % g.R
    Z = g.n_sink
    for b in range(g.B):
        for h in range(g.H):
            for s in range(Z):
                if plen[b, h, s] > 0:
                    keep[b, h, s] = True
                else:
                    admit[b, h, s] = True
            cands = [(-float(mass[b, h, s]), 0, s) for s in range(Z, g.S) if plen[b, h, s] > 0]
            cands += [(-float(mass[b, h, g.S + old * g.n_qblk + e]), 1, e) for e in range(g.n_qblk)
                      if not (e < Z and plen[b, h, e] == 0)]
            cands.sort()
            for _, kind, idx in cands[: g.S - Z]:
                if kind == 0:
                    keep[b, h, idx] = True
                else:
                    admit[b, h, idx] = True
    return keep, admit


def apply_update(state: dict, keep, admit, k_l, v_l, kbar_l, ring_head: int, step_id: int,
                 g: Geometry) -> dict:
    """Move admitted blocks into vacated slots (reading R13) and return the new state.

    Vacated slots = empty or dropped slots, ascending; admitted blocks in
    ascending order fill them pairwise.  With sink slots (R20) an empty sink
    slot s takes admitted block s, and pairing uses the other slots and
    blocks only.  A filled slot gets the block's rows
    (raster order within the block), zero padding, len = block size,
    src = step_id * n_qblk + e and kbar = the block's pooled key.  Vacated
    slots left over are emptied (rows zero, len 0, src EMPTY_SRC, kbar 0).
    """
    k_p = state["k_p"].copy()
    v_p = state["v_p"].copy()
    plen = state["persist_len"].copy()
    src = state["persist_src"].copy()
    kbar = state["persist_kbar"].copy()
    n_rep = np.zeros((g.B, g.H), dtype=np.int32)
    old = ring_head % g.R
    Z = g.n_sink
    for b in range(g.B):
        for h in range(g.H):
            fills = [s for s in range(Z) if plen[b, h, s] == 0]
            assert all(admit[b, h, s] for s in fills) and all(keep[b, h, s] for s in range(Z) if s not in fills)
            vac = [s for s in range(Z, g.S) if not (plen[b, h, s] > 0 and keep[b, h, s])]
            ent = [e for e in range(g.n_qblk) if admit[b, h, e] and e not in fills]
            assert len(ent) <= len(vac)
            n_rep[b, h] = len(ent) + len(fills)
            pairs = list(zip(fills, fills)) + [(s, ent[j] if j < len(ent) else None) for j, s in enumerate(vac)]
            for s, e in pairs:
                k_p[b, h, s] = 0
                v_p[b, h, s] = 0
                if e is not None:
                    tok = old * g.chunk_tokens + g.block_tok[e]
                    n = len(tok)
                    k_p[b, h, s, :n] = k_l[b, h, tok]
                    v_p[b, h, s, :n] = v_l[b, h, tok]
                    plen[b, h, s] = n
                    src[b, h, s] = step_id * g.n_qblk + e
                    kbar[b, h, s] = kbar_l[b, h, old * g.n_qblk + e]
                else:
                    plen[b, h, s] = 0
                    src[b, h, s] = EMPTY_SRC
                    kbar[b, h, s] = 0
    return dict(k_p=k_p, v_p=v_p, persist_len=plen, persist_src=src, persist_kbar=kbar,
                n_replaced=n_rep, ring_head=(ring_head + 1) % g.R)


def persist_update(state: dict, mass, k_l, v_l, kbar_l, ring_head: int, step_id: int,
                   g: Geometry) -> dict:
    """Decide (update_decisions) then move data (apply_update)."""
    keep, admit = update_decisions(mass, state["persist_len"], ring_head, g)
    out = apply_update(state, keep, admit, k_l, v_l, kbar_l, ring_head, step_id, g)
    out["keep"] = keep
    out["admit"] = admit
    return out


# ----------------------------------------------------------------------------
# The local ring and the per-chunk schedule (review page, the paper's
# training-algorithm fragment: every denoising step applies PBSA with top-K to
# the current chunk; the t=0 cache pass applies PBSA with top-K and updates
# the persistent (P) and local (L) caches; readings R9, R10, R21)
# ----------------------------------------------------------------------------


def ring_append(k_l, v_l, k_new, v_new, ring_head: int, g: Geometry):
    """Local ring with the current chunk's keys and values in its newest slot.

    The ring holds R chunks; physical chunk slot ``ring_head`` is the oldest,
    so the newest is slot (ring_head + R - 1) mod R -- the slot the previous
    update evicted.  Returns new arrays; the other slots are unchanged.
    """
    k = k_l.copy()
    v = v_l.copy()
    c = (ring_head + g.R - 1) % g.R
    rows = slice(c * g.chunk_tokens, (c + 1) * g.chunk_tokens)
    k[:, :, rows] = k_new
    v[:, :, rows] = v_new
    return k, v


def decode_chunk(state: dict, k_l, v_l, passes, ring_head: int, step_id: int, g: Geometry,
                 mass: str = "pooled", qblocks=None) -> dict:
    """One generated chunk: its denoising passes, then the cache pass.

    ``passes`` is a list of (q, k, v) of the chunk, one per pass; the last
    entry is the cache pass (t = 0), the ones before it the denoising passes
    (reading R21: their number is the caller's).  Every pass writes its own
    keys and values into the newest ring slot, so the local window it scores
    and attends holds the previous chunks and the current chunk (R3); the
    denoising passes only attend; the cache pass attends and then updates
    the persistent cache with its own masses, evicting the oldest ring chunk
    (R9, R10).  ``state`` holds k_p, v_p, persist_len, persist_src,
    persist_kbar.  Returns per-pass selections, O and LSE (``qblocks``
    restricts the attention rows, as in ``attend``), the ring after the
    chunk and the updated state.
    """
    out = []
    for i, (q, k, v) in enumerate(passes):
        k_l, v_l = ring_append(k_l, v_l, k, v, ring_head, g)
        sel = score_select(q, k_l, ring_head, state["persist_kbar"], state["persist_len"], g)
        tm = None
        if mass == "token" and i == len(passes) - 1:
            tm = token_mass(q, state["k_p"], state["persist_len"], k_l, sel["topk_idx"], g)
        O, L = attend(q, state["k_p"], state["v_p"], state["persist_len"], k_l, v_l, sel["topk_idx"], g,
                      qblocks=qblocks)
        out.append(dict(sel=sel, O=O, L=L, token_mass=tm))
    last = out[-1]
    m = last["sel"]["mass"] if mass == "pooled" else last["token_mass"]
    up = persist_update(state, m, k_l, v_l, last["sel"]["kbar_l"], ring_head, step_id, g)
    return dict(passes=out, k_l=k_l, v_l=v_l, update=up, mass=m)


# ----------------------------------------------------------------------------
# Near-tie accounting (reading R15)
# ----------------------------------------------------------------------------


def near_tie_rows(scores_row: np.ndarray, k: int, rel: float = 1e-4):
    """Band around the k-th/(k+1)-th boundary of one row of oracle scores.

    Returns (is_near_tie, band, boundary): the row is a near tie when the gap
    between the k-th and (k+1)-th largest score is below rel * (max - min).
    Elements whose score lies within ``band`` of the boundary may legitimately
    be swapped by a different summation order.
    """
    s = np.sort(scores_row.astype(np.float64))[::-1]
    if k >= len(s):
        return False, 0.0, -np.inf
    band = rel * float(s[0] - s[-1])
    boundary = 0.5 * float(s[k - 1] + s[k])
    return bool(s[k - 1] - s[k] < band), band, boundary
