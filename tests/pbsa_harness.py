"""Helpers shared by the GPU parity tests: upload seeded inputs, run the HIP
path through the C ABI, and compare with the oracle (with near-tie accounting
for the integer decisions that floating point takes)."""
from __future__ import annotations

import numpy as np
import torch

import block_sparse_attention_15_amd as pb
import oracle


def dev(x: np.ndarray, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


class GpuStep:
    """Device buffers of one decode step, filled from a synth input dict."""

    def __init__(self, cfg: dict, x: dict):
        self.cfg = cfg
        self.p = pb.pbsa_plan(cfg)
        p, s = self.p, pb.shapes(self.p)
        dt = p.torch_dtype
        self.q = dev(x["q"], dt)
        self.k_l = dev(x["k_l"], dt)
        self.v_l = dev(x["v_l"], dt)
        self.k_p = dev(x["k_p"], dt)
        self.v_p = dev(x["v_p"], dt)
        self.plen = dev(x["persist_len"])
        self.psrc = dev(x["persist_src"])
        self.ring_head = dev(x["ring_head"])
        self.step_counter = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.pkbar = torch.empty(s["persist_kbar"], dtype=torch.float32, device="cuda")
        self.topk = torch.full(s["topk_idx"], -7, dtype=torch.int32, device="cuda")
        self.mass = torch.full(s["mass"], float("nan"), dtype=torch.float32, device="cuda")
        self.kbar_l = torch.full(s["kbar_local"], float("nan"), dtype=torch.float32, device="cuda")
        self.o = torch.full(s["q"], float("nan"), dtype=dt, device="cuda")
        self.lse = torch.full(s["lse"], float("nan"), dtype=torch.float32, device="cuda")
        self.n_rep = torch.full(s["n_replaced"], -1, dtype=torch.int32, device="cuda")
        self.ws_score = pb.workspace(p, "score_select")
        self.ws_bwd = pb.workspace(p, "bwd")
        self.ws_update = pb.workspace(p, "persist_update")
        self.ws_fwd = pb.workspace(p, "fwd")
        pb.pbsa_pool_slots(p, self.k_p, self.plen, self.pkbar)
        pb.pbsa_pool_local(p, self.k_l, self.kbar_l)   # the ring was written from outside the library

    def score_select(self):
        pb.pbsa_score_select(self.p, self.q, self.kbar_l, self.ring_head, self.pkbar, self.plen, self.topk, self.mass,
                             self.ws_score)

    def fwd(self, topk=None):
        pb.pbsa_fwd(self.p, self.q, self.k_p, self.v_p, self.plen, self.k_l, self.v_l,
                    self.topk if topk is None else topk, self.o, self.lse, self.ws_fwd)

    def fwd_mass(self, topk=None):
        """Forward plus token-exact masses (into self.mass)."""
        if not hasattr(self, "ws_fwd_mass"):
            self.ws_fwd_mass = pb.workspace(self.p, "fwd_mass")
        pb.pbsa_fwd_mass(self.p, self.q, self.k_p, self.v_p, self.plen, self.k_l, self.v_l,
                         self.topk if topk is None else topk, self.o, self.lse, self.mass, self.ws_fwd_mass)

    def bwd(self, dout, topk=None):
        s = pb.shapes(self.p)
        f = dict(dtype=torch.float32, device="cuda")
        g = dict(dq=torch.full(s["q"], float("nan"), **f), dk_p=torch.full(s["k_pers"], float("nan"), **f),
                 dv_p=torch.full(s["k_pers"], float("nan"), **f), dk_l=torch.full(s["k_local"], float("nan"), **f),
                 dv_l=torch.full(s["k_local"], float("nan"), **f))
        pb.pbsa_bwd(self.p, self.q, self.k_p, self.v_p, self.plen, self.k_l, self.v_l,
                    self.topk if topk is None else topk, self.o, self.lse, dout, g["dq"], g["dk_p"], g["dv_p"],
                    g["dk_l"], g["dv_l"], self.ws_bwd)
        return g

    def update(self, step_id: int, mass=None):
        self.step_counter.fill_(step_id)
        pb.pbsa_persist_update(self.p, self.mass if mass is None else mass, self.k_l, self.v_l, self.kbar_l,
                               self.ring_head, self.step_counter, self.k_p, self.v_p, self.plen, self.psrc,
                               self.pkbar, self.n_rep, self.ws_update)

    def state(self) -> dict:
        return dict(k_p=host(self.k_p), v_p=host(self.v_p), persist_len=host(self.plen),
                    persist_src=host(self.psrc), persist_kbar=host(self.pkbar), ring_head=int(host(self.ring_head)[0]))


def compare_topk(gpu_idx: np.ndarray, ora_idx: np.ndarray, scores: np.ndarray, k: int, rel=1e-4):
    """Rows must match as sets, except near-tie rows whose differing blocks all lie in the band.

    Returns (n_near_tie_rows, n_mismatched_rows).  Raises AssertionError on a
    mismatch that is not a near tie.
    """
    B, H, NQ, _ = gpu_idx.shape
    n_band = n_mis = 0
    for b in range(B):
        for h in range(H):
            for i in range(NQ):
                row = scores[b, h, i]
                nt, band, boundary = oracle.near_tie_rows(row, k, rel)
                n_band += nt
                a, o = set(gpu_idx[b, h, i].tolist()), set(ora_idx[b, h, i].tolist())
                assert len(a) == k and all(0 <= v < row.shape[0] for v in a), (b, h, i, sorted(a))
                assert list(gpu_idx[b, h, i]) == sorted(a), "ids not ascending"
                if a == o:
                    continue
                n_mis += 1
                diff = a ^ o
                assert nt and all(abs(float(row[p]) - boundary) <= band for p in diff), \
                    (b, h, i, sorted(a - o), sorted(o - a), [float(row[p]) for p in diff], boundary, band)
    return n_band, n_mis


def decisions_from_state(before: dict, after: dict, step_id: int, nq: int):
    """Keep/admit decisions implied by a GPU update (src ids are unique per step)."""
    keep = (before["persist_len"] > 0) & (after["persist_src"] == before["persist_src"])
    B, H, S = keep.shape
    admit = np.zeros((B, H, nq), dtype=bool)
    base = step_id * nq
    for b in range(B):
        for h in range(H):
            for v in after["persist_src"][b, h]:
                if base <= v < base + nq:
                    admit[b, h, v - base] = True
    return keep, admit


def compare_update_decisions(keep_g, admit_g, keep_o, admit_o, mass_o, plen_before, ring_head, g, rel=1e-4):
    """Decision differences must be near ties of the oracle's masses; returns #heads that differ."""
    n_diff = 0
    old = ring_head % g.R
    for b in range(g.B):
        for h in range(g.H):
            if (keep_g[b, h] == keep_o[b, h]).all() and (admit_g[b, h] == admit_o[b, h]).all():
                continue
            n_diff += 1
            vals = [float(mass_o[b, h, s]) for s in range(g.S) if plen_before[b, h, s] > 0]
            vals += [float(mass_o[b, h, g.S + old * g.n_qblk + e]) for e in range(g.n_qblk)]
            nt, band, boundary = oracle.near_tie_rows(np.array(vals), g.S, rel)
            changed = [float(mass_o[b, h, s]) for s in np.nonzero(keep_g[b, h] != keep_o[b, h])[0]]
            changed += [float(mass_o[b, h, g.S + old * g.n_qblk + e]) for e in np.nonzero(admit_g[b, h] != admit_o[b, h])[0]]
            assert nt and all(abs(v - boundary) <= band for v in changed), (b, h, changed, boundary, band)
    return n_diff


def rel_l2(a: np.ndarray, b: np.ndarray) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))
