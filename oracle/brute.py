"""Brute-force PBSA in pure-Python float64 loops, for tiny shapes only (test infrastructure).

An independent second writing of the same definitions as ``oracle.pbsa`` (same
pages, same readings), used to pin the vectorised oracle: block membership is
found by scanning every token's (row, column) against the block grid, scores
are explicit dot products, the top-k is an explicit sort with the tie rule,
softmax is summed term by term, and the update ranks candidates exhaustively.
No numpy linear algebra is used.
"""
from __future__ import annotations

import math


def _blocks_of_frame(fh, fw, bh, bw):
    """Block id of each token of one frame (block-row-major), by scanning tokens."""
    ncols = (fw + bw - 1) // bw
    owner = []
    for r in range(fh):
        for c in range(fw):
            owner.append((r // bh) * ncols + (c // bw))
    nblk = ((fh + bh - 1) // bh) * ncols
    members = [[] for _ in range(nblk)]
    for t, o in enumerate(owner):
        members[o].append(t)          # raster order within each block
    return members


def chunk_blocks(fh, fw, bh, bw, chunk_frames):
    """Token lists (offsets inside a chunk) of each block of a chunk, block_t = 1."""
    per = _blocks_of_frame(fh, fw, bh, bw)
    out = []
    for f in range(chunk_frames):
        for m in per:
            out.append([f * fh * fw + t for t in m])
    return out


def _dot(a, b):
    s = 0.0
    for x, y in zip(a, b):
        s += x * y
    return s


def _mean(rows):
    n = len(rows)
    d = len(rows[0])
    return [sum(r[j] for r in rows) / n for j in range(d)]


def step(cfg, q, k_l, v_l, k_p, v_p, plen, ring_head, step_id):
    """One decode step for batch 0 of every head; inputs are nested lists / arrays.

    Returns dict with per-head lists: topk (physical ids ascending), O rows,
    LSE, mass (slot s, then S + physical local block), and the updated slot
    contents (len, src, rows of K and V).
    """
    fh, fw, bh, bw = cfg["frame_h"], cfg["frame_w"], cfg["block_h"], cfg["block_w"]
    cf = cfg["chunk_frames"]
    blocks = chunk_blocks(fh, fw, bh, bw, cf)
    nq = len(blocks)
    ct = cf * fh * fw
    R = cfg["local_cache_size"] // ct
    nl = R * nq
    S = len(plen[0][0])
    D = cfg["head_dim"]
    scale = 1.0 / math.sqrt(D)
    if cfg.get("use_local_block_sparse_attn", 1):
        k = max(1, min(nl, math.ceil(cfg["topk_ratio"] * nl - 1e-6)))
    else:
        k = nl
    H = cfg["heads"]
    res = dict(topk=[], O=[], LSE=[], mass=[], slots=[], n_replaced=[])
    for h in range(H):
        Q = [list(map(float, row)) for row in q[0][h]]
        KL = [list(map(float, row)) for row in k_l[0][h]]
        VL = [list(map(float, row)) for row in v_l[0][h]]
        lens = [int(x) for x in plen[0][h]]
        KP = [[list(map(float, r)) for r in k_p[0][h][s]] for s in range(S)]
        VP = [[list(map(float, r)) for r in v_p[0][h][s]] for s in range(S)]
        # local block tokens, physical id p = chunk_slot * nq + blk
        ltok = [[(p // nq) * ct + t for t in blocks[p % nq]] for p in range(nl)]
        logical = [(((p // nq) - ring_head) % R) * nq + p % nq for p in range(nl)]
        qbar = [_mean([Q[t] for t in blocks[i]]) for i in range(nq)]
        kbar = [_mean([KL[t] for t in ltok[p]]) for p in range(nl)]
        pbar = [(_mean(KP[s][:lens[s]]) if lens[s] else None) for s in range(S)]
        # top-k: explicit sort by (-score, logical index)
        topk = []
        for i in range(nq):
            sc = [(-scale * _dot(qbar[i], kbar[p]), logical[p], p) for p in range(nl)]
            sc.sort()
            topk.append(sorted(x[2] for x in sc[:k]))
        res["topk"].append(topk)
        # attention, term by term
        O = [None] * ct
        LSE = [None] * ct
        for i in range(nq):
            keys = []
            for s in range(S):
                for r in range(lens[s]):
                    keys.append((KP[s][r], VP[s][r]))
            for p in topk[i]:
                for t in ltok[p]:
                    keys.append((KL[t], VL[t]))
            for t in blocks[i]:
                logits = [scale * _dot(Q[t], kk) for kk, _ in keys]
                m = max(logits)
                w = [math.exp(x - m) for x in logits]
                z = sum(w)
                O[t] = [sum(w[j] * keys[j][1][d] for j in range(len(keys))) / z for d in range(D)]
                LSE[t] = m + math.log(z)
        res["O"].append(O)
        res["LSE"].append(LSE)
        # pooled masses
        mass = [0.0] * (S + nl)
        for i in range(nq):
            cand = [(s, scale * _dot(qbar[i], pbar[s])) for s in range(S) if lens[s]]
            cand += [(S + p, scale * _dot(qbar[i], kbar[p])) for p in range(nl)]
            m = max(x[1] for x in cand)
            z = sum(math.exp(x[1] - m) for x in cand)
            for j, x in cand:
                mass[j] += math.exp(x - m) / z
        res["mass"].append(mass)
        # update: exhaustive ranking of all candidates; pinned sink slots
        # (the first `sink` slots) stay, or take the evicted block of their index
        old = ring_head % R
        sink = cfg.get("sink_slots", 0)
        pinned = {s for s in range(sink) if lens[s]}
        sink_fill = {s: s for s in range(sink) if not lens[s]}
        cands = [(-mass[s], 0, s) for s in range(S) if lens[s] and s not in pinned]
        cands += [(-mass[S + old * nq + e], 1, e) for e in range(nq) if e not in sink_fill]
        cands.sort()
        kept = cands[:S - sink]
        keep = {c[2] for c in kept if c[1] == 0} | pinned
        admit = sorted(c[2] for c in kept if c[1] == 1)
        vac = [s for s in range(S) if s not in keep and s not in sink_fill]
        slots = []
        ent_for = dict(zip(vac, admit))
        ent_for.update(sink_fill)
        for s in range(S):
            if s in keep:
                slots.append((lens[s], None, [r[:] for r in KP[s]], [r[:] for r in VP[s]]))
            elif s in ent_for:
                e = ent_for[s]
                tok = [old * ct + t for t in blocks[e]]
                kr = [KL[t][:] for t in tok] + [[0.0] * D] * (len(KP[s]) - len(tok))
                vr = [VL[t][:] for t in tok] + [[0.0] * D] * (len(KP[s]) - len(tok))
                slots.append((len(tok), step_id * nq + e, kr, vr))
            else:
                slots.append((0, "empty", [[0.0] * D] * len(KP[s]), [[0.0] * D] * len(KP[s])))
        res["slots"].append(slots)
        res["n_replaced"].append(len(admit) + len(sink_fill))
    return res
