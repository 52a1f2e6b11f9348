"""Benchmark of the PBSA decode step at the 12-head, d=128 decode shape on one MI355X.

Headline: one decode step = the whole inference hot path over one chunk --
append the chunk's K/V to the local ring, pooled scoring + top-k selection +
pooled masses, the sparse attention forward, and the persistent-cache update
(which also advances the ring) -- timed end to end with HIP events on the one
stream every call uses.  ``value`` is its effective TFLOP/s: 4*d flops per
attended (query, key) pair, pairs counted exactly by a deterministic untimed
replay that reads back the selections and slot lengths.  The cache state
rolls from step to step as in a rollout.

Extra keys: per-op HIP-event times (warm, and cold with a cache-evicting fill
before every op), the training step (the decode step plus the backward),
the same decode step with [3,4,4] blocks, an 80-chunk graph-replayed
rollout and the per-chunk schedule with denoising passes, and the oracle leg:
the CPU oracle timed on the same decode step (all heads) plus its parity
counts (near ties and selection mismatches at the decode shape, and the
cumulative selection-mismatch count of the 80-chunk rollout checked
teacher-forced).

Prints one JSON line.  Only one GPU is supported: the method is independent
per head, so a multi-GPU run would shard heads with no exchange.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MI355X_BF16_TFLOPS = 2516.6   # dense bf16 MFMA peak (256 CU x 2.4 GHz x 4096 flop/clk)
MI355X_HBM_GBS = 8000.0        # HBM3E peak
DECODE_OPS = ("append", "score_select", "fwd", "update")
TRAIN_OPS = ("append", "score_select", "fwd", "bwd", "update")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_c1")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle leg (CPU baseline and parity counts)")
    ap.add_argument("--no-train", action="store_true", help="skip the training-step timing")
    ap.add_argument("--no-344", action="store_true", help="skip the [3,4,4]-block decode step")
    ap.add_argument("--cpu-heads", type=int, default=12, help="heads in the CPU oracle sample")
    ap.add_argument("--rollout-steps", type=int, default=80,
                    help="chunks of the graph-replayed rollout (0 skips it)")
    ap.add_argument("--cold-steps", type=int, default=5,
                    help="extra steps with a cache-evicting fill before every op (0 skips them)")
    ap.add_argument("--denoise-passes", type=int, default=4,
                    help="denoising passes per chunk in the schedule timing (the pages do not give it)")
    return ap.parse_args()


def _ev():
    import torch
    return torch.cuda.Event(enable_timing=True)


_T0 = time.perf_counter()


def progress(msg: str):
    print(f"[bench {time.perf_counter() - _T0:6.1f}s] {msg}", file=sys.stderr, flush=True)


class Bench:
    """Device buffers of the decode step at one workload, with a rolling cache state."""

    def __init__(self, cfg):
        import torch
        import block_sparse_attention_15_amd as pb
        import synth
        self.torch, self.pb = torch, pb
        self.cfg = cfg
        self.p = pb.pbsa_plan(cfg)
        p, s = self.p, pb.shapes(self.p)
        x = synth.make_step_inputs(cfg)
        dout = synth.make_dout(dict(cfg, dout_seed=3))
        dt = p.torch_dtype
        dev = lambda a, d=None: (torch.from_numpy(np.ascontiguousarray(a)).to(d) if d else
                                 torch.from_numpy(np.ascontiguousarray(a))).cuda()
        self.pristine = dict(k_p=dev(x["k_p"], dt), v_p=dev(x["v_p"], dt), plen=dev(x["persist_len"]),
                             psrc=dev(x["persist_src"]), ring_head=dev(x["ring_head"]), k_l=dev(x["k_l"], dt),
                             v_l=dev(x["v_l"], dt), step=torch.zeros(1, dtype=torch.int32, device="cuda"))
        self.live = {k: v.clone() for k, v in self.pristine.items()}
        self.pkbar0 = torch.empty(s["persist_kbar"], dtype=torch.float32, device="cuda")
        pb.pbsa_pool_slots(p, self.pristine["k_p"], self.pristine["plen"], self.pkbar0)
        self.pkbar = self.pkbar0.clone()
        self.kbar_l0 = torch.empty(s["kbar_local"], dtype=torch.float32, device="cuda")
        pb.pbsa_pool_local(p, self.pristine["k_l"], self.kbar_l0)
        self.kbar_l = self.kbar_l0.clone()
        self.q = dev(x["q"], dt)
        # the chunk appended each step: the current chunk of the input ring
        nq = p.chunk_tokens
        self.k_new = self.pristine["k_l"][:, :, nq:2 * nq].contiguous()
        self.v_new = self.pristine["v_l"][:, :, nq:2 * nq].contiguous()
        self.dout = dev(dout, dt)
        f32 = dict(dtype=torch.float32, device="cuda")
        self.topk = torch.empty(s["topk_idx"], dtype=torch.int32, device="cuda")
        self.mass = torch.empty(s["mass"], **f32)
        self.o = torch.empty(s["q"], dtype=dt, device="cuda")
        self.lse = torch.empty(s["lse"], **f32)
        self.grads = None
        self.n_rep = torch.empty(s["n_replaced"], dtype=torch.int32, device="cuda")
        self.ws_s = pb.workspace(p, "score_select")
        self.ws_u = pb.workspace(p, "persist_update")
        self.ws_f = pb.workspace(p, "fwd")
        self.ws_b = None
        self.step_id = 0
        self._bl = self.block_lens().astype(np.int64)

    def enable_train(self):
        torch, s = self.torch, self.pb.shapes(self.p)
        f32 = dict(dtype=torch.float32, device="cuda")
        self.grads = dict(dq=torch.empty(s["q"], **f32), dk_p=torch.empty(s["k_pers"], **f32),
                          dv_p=torch.empty(s["k_pers"], **f32), dk_l=torch.empty(s["k_local"], **f32),
                          dv_l=torch.empty(s["k_local"], **f32))
        self.ws_b = self.pb.workspace(self.p, "bwd")

    def reset(self):
        for k, v in self.pristine.items():
            self.live[k].copy_(v)
        self.pkbar.copy_(self.pkbar0)
        self.kbar_l.copy_(self.kbar_l0)
        self.step_id = 0

    def ops(self, train=False):
        pb, L, p = self.pb, self.live, self.p
        out = [("append", lambda: pb.pbsa_ring_append(p, self.k_new, self.v_new, L["ring_head"], L["k_l"], L["v_l"],
                                                     self.kbar_l)),
               ("score_select", lambda: pb.pbsa_score_select(p, self.q, self.kbar_l, L["ring_head"], self.pkbar,
                                                             L["plen"], self.topk, self.mass, self.ws_s)),
               ("fwd", lambda: pb.pbsa_fwd(p, self.q, L["k_p"], L["v_p"], L["plen"], L["k_l"], L["v_l"], self.topk,
                                           self.o, self.lse, self.ws_f))]
        if train:
            G = self.grads
            out.append(("bwd", lambda: pb.pbsa_bwd(p, self.q, L["k_p"], L["v_p"], L["plen"], L["k_l"], L["v_l"],
                                                   self.topk, self.o, self.lse, self.dout, G["dq"], G["dk_p"],
                                                   G["dv_p"], G["dk_l"], G["dv_l"], self.ws_b)))
        out.append(("update", lambda: pb.pbsa_persist_update(p, self.mass, L["k_l"], L["v_l"], self.kbar_l,
                                                             L["ring_head"], L["step"], L["k_p"], L["v_p"], L["plen"],
                                                             L["psrc"], self.pkbar, self.n_rep, self.ws_u)))
        return out

    def step(self, train=False, ev=None, flush=None, record=None):
        """One step.  ``ev``: dict op -> (start, end) events to record;
        ``flush``: callable run before each op (outside its events) to evict
        the caches for cold-HBM timing; ``record``: list that receives the
        step's exact work (untimed)."""
        for name, fn in self.ops(train):
            if name == "update" and record is not None:
                record.append(self.account())
                plen_before = self.live["plen"].cpu().numpy()
            if flush is not None:
                flush()
            if ev is not None:
                ev[name][0].record()
            fn()
            if ev is not None:
                ev[name][1].record()
        if record is not None:
            record[-1]["update_bytes"] = self.update_bytes(plen_before)
        self.step_id += 1

    # -- exact work accounting (untimed replay) --------------------------------
    def block_lens(self):
        """Token count of each block of a chunk (block-row-major tiling, smaller edge blocks)."""
        c = self.cfg
        out = []
        for _ in range(0, c["chunk_frames"], c["block_t"]):
            for r0 in range(0, c["frame_h"], c["block_h"]):
                for c0 in range(0, c["frame_w"], c["block_w"]):
                    out.append(c["block_t"] * min(c["block_h"], c["frame_h"] - r0) *
                               min(c["block_w"], c["frame_w"] - c0))
        return np.array(out)

    def account(self):
        """Attended (query, key) pairs of the current selection and slot lengths."""
        p = self.p
        topk = self.topk.cpu().numpy()
        plen = self.live["plen"].cpu().numpy().astype(np.int64)
        bl = self._bl
        nq = p.blocks_per_chunk
        pers = plen.sum(-1)                                   # [B,H] valid persistent tokens
        loc = bl[topk % nq].sum(-1)                           # [B,H,nq] selected local tokens
        pairs = (bl[None, None, :] * (pers[..., None] + loc)).sum()
        return dict(pairs=int(pairs), pers_tokens=float(pers.mean()), local_tokens=float(loc.mean()))

    def update_bytes(self, plen_before):
        """HBM bytes the update moved: each admitted block reads its len rows of K
        and V and writes the slot's C rows (data + zero padding); each emptied
        slot writes C zero rows of K and V."""
        p = self.p
        src = self.live["psrc"].cpu().numpy().astype(np.int64)
        plen = self.live["plen"].cpu().numpy()
        esz = 2 if self.cfg["dtype"] == "bf16" else 4
        row = p.D * esz
        base = self.step_id * p.blocks_per_chunk
        ent = (src >= base) & (src < base + p.blocks_per_chunk)
        lens = self._bl[np.where(ent, src - base, 0)] * ent
        emptied = (plen == 0) & (plen_before > 0)
        return float(2 * row * (lens.sum() + p.slot_rows * (ent.sum() + emptied.sum())))

    def score_bytes(self):
        """Bytes score_select moves: the queries (pooled in the call), the pooled
        keys of the local blocks and slots (ring and slot metadata, pooled when
        their keys were written), the selections and the masses."""
        p, esz = self.p, (2 if self.cfg["dtype"] == "bf16" else 4)
        nl = p.local_blocks
        return p.B * p.H * (p.chunk_tokens * p.D * esz + (nl + p.persistent_slots) * p.D * 4 +
                            p.blocks_per_chunk * p.topk * 4 + (nl + p.persistent_slots) * 4)

    def append_bytes(self):
        """The chunk's keys and values read and written once, plus its pooled keys."""
        p, esz = self.p, (2 if self.cfg["dtype"] == "bf16" else 4)
        return 2 * 2 * p.B * p.H * p.chunk_tokens * p.D * esz + p.B * p.H * p.blocks_per_chunk * p.D * 4


def _stats(t):
    t = np.asarray(t)
    return dict(mean=float(t.mean()), p50=float(np.median(t)), p99=float(np.percentile(t, 99)))


def time_steps(b, steps, warmup, train=False, cold_steps=0):
    """The step timed end to end (no events inside), then per-op events over
    the same number of steps, then cold per-op events, then the exact work of
    a replay of the timed steps from the same starting state."""
    import torch
    ops = TRAIN_OPS if train else DECODE_OPS
    b.reset()
    for _ in range(warmup):
        b.step(train)
    torch.cuda.synchronize()
    e0, e1 = _ev(), _ev()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        b.step(train)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    span_ms = e0.elapsed_time(e1)
    # per-op events
    evs = [{op: (_ev(), _ev()) for op in ops} for _ in range(steps)]
    for k in range(steps):
        b.step(train, ev=evs[k])
    torch.cuda.synchronize()
    per_op = {op: _stats([e[op][0].elapsed_time(e[op][1]) for e in evs]) for op in ops}
    cold = None
    if cold_steps > 0:
        junk = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        cevs = [{op: (_ev(), _ev()) for op in ops} for _ in range(cold_steps)]
        for k in range(cold_steps):
            b.step(train, ev=cevs[k], flush=lambda: junk.fill_(k & 0xFF))
        torch.cuda.synchronize()
        cold = {op: _stats([e[op][0].elapsed_time(e[op][1]) for e in cevs]) for op in ops}
        del junk
    # exact accounting: replay warmup + timed steps from the same state
    b.reset()
    for _ in range(warmup):
        b.step(train)
    rec = []
    for _ in range(steps):
        b.step(train, record=rec)
    torch.cuda.synchronize()
    return dict(ms=span_ms / steps, wall=wall, per_op=per_op, cold=cold, acc=rec)


def traffic_record(workload: str):
    """HBM bytes per launch of each op, from the committed FETCH_SIZE /
    WRITE_SIZE summary of this workload.  Returns {} when there is none or
    when the kernel sources changed since the counters were taken."""
    from block_sparse_attention_15_amd.build import source_digest
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.txt")
    if not os.path.exists(path):
        return {}
    digest, out = None, {}
    for line in open(path):
        f = line.split()
        if len(f) >= 2 and f[0] == "source_digest:":
            digest = f[1]
        elif len(f) >= 3 and f[0] == "traffic":
            out[f[1]] = float(f[2])
    return out if digest == source_digest() else {}


def summarize(b, r, ops):
    """Per-op dict with times, rates and bytes; plus pairs and the step's flops."""
    p = b.p
    pairs = float(np.mean([a["pairs"] for a in r["acc"]]))
    kern = {op: {"ms": round(v["mean"], 4), "p50_ms": round(v["p50"], 4), "p99_ms": round(v["p99"], 4)}
            for op, v in r["per_op"].items()}
    fwd_flops = 4 * p.D * pairs
    kern["fwd"].update(tflops=round(fwd_flops / (r["per_op"]["fwd"]["mean"] * 1e-3) / 1e12, 2),
                       gflop=round(fwd_flops / 1e9, 2))
    if "bwd" in kern:
        bwd_flops = 10 * p.D * pairs
        kern["bwd"].update(tflops=round(bwd_flops / (r["per_op"]["bwd"]["mean"] * 1e-3) / 1e12, 2),
                           gflop=round(bwd_flops / 1e9, 2))
    ub = float(np.mean([a["update_bytes"] for a in r["acc"]]))
    hbm = dict(append=b.append_bytes(), score_select=b.score_bytes(), update=ub)
    for op, nbytes in hbm.items():
        kern[op].update(gbs=round(nbytes / (r["per_op"][op]["mean"] * 1e-3) / 1e9, 1), mb=round(nbytes / 1e6, 2))
    cold = None
    if r["cold"]:
        cold = {}
        for op in ops:
            c = {"ms": round(r["cold"][op]["mean"], 4), "p50_ms": round(r["cold"][op]["p50"], 4)}
            if op in hbm:
                c["gbs"] = round(hbm[op] / (r["cold"][op]["mean"] * 1e-3) / 1e9, 1)
                c["frac_hbm"] = round(c["gbs"] / MI355X_HBM_GBS, 4)
            cold[op] = c
    return kern, cold, pairs


def run_rollout(steps: int, denoise: int, keep_states: bool):
    """Long rollout: chunk s's q/k/v (seeded, drifting planted blocks) are staged
    into the loop's buffers (device-to-device) and one captured graph runs the
    cache pass (ring append, score/select, fwd, persistent update); only the
    replays are timed.  Also times the per-chunk schedule with ``denoise``
    denoising passes before the cache pass, each pass with its own inputs
    (the next chunks of the seeded stream stand in for the noisy inputs), and
    the graph with token-exact masses.  With ``keep_states``, the graph run
    keeps every step's pre-step slot metadata and ring head and its
    selection, for the oracle leg's teacher-forced check."""
    import torch
    import block_sparse_attention_15_amd as pb
    from block_sparse_attention_15_amd.rollout import DecodeLoop
    import synth
    rcfg = synth.workload("rollout_c4", steps=steps)
    stream = synth.RolloutStream(rcfg)
    x = synth.make_step_inputs(dict(rcfg, plant_frac=0.0))
    p = pb.pbsa_plan(rcfg)
    dt = p.torch_dtype
    dev = lambda a: torch.from_numpy(a).to(dt).cuda()
    chunks = []
    for s in range(-1, steps):
        chunks.append(stream.chunk(s))
        if s % 20 == 19:
            progress(f"rollout inputs: {s + 2} chunks")
    dq = torch.stack([dev(c["q"]) for c in chunks[1:]])
    dk = torch.stack([dev(c["k"]) for c in chunks[1:]])
    dv = torch.stack([dev(c["v"]) for c in chunks[1:]])

    def fresh(mass="pooled", nd=0):
        cache = pb.PBSACache(p)
        cache.k_pers.copy_(dev(x["k_p"]))
        cache.v_pers.copy_(dev(x["v_p"]))
        cache.persist_len.copy_(torch.from_numpy(x["persist_len"]).cuda())
        cache.persist_src.copy_(torch.from_numpy(x["persist_src"]).cuda())
        ct = p.chunk_tokens
        cache.k_local[:, :, :ct].copy_(dev(chunks[0]["k"]))
        cache.v_local[:, :, :ct].copy_(dev(chunks[0]["v"]))
        cache.refresh_pooled_keys()
        return cache, DecodeLoop(p, cache, mass=mass, denoise_passes=nd)

    def stage(loop, s):
        n = loop.denoise_passes
        for i in range(n + 1):
            j = s if i == n else (s + 1 + i) % steps   # cache pass: chunk s; denoising passes: later chunks
            loop.load_pass(i, dq[j], dk[j], dv[j])

    out = {"steps": steps, "denoise_passes": denoise}
    states = []
    for mode in ("eager", "graph", "schedule", "token_graph"):
        mass = "token" if mode == "token_graph" else "pooled"
        nd = denoise if mode == "schedule" else 0
        cache, loop = fresh(mass, nd)
        if mode != "eager":
            _, warm = fresh(mass, nd)
            stage(warm, 0)
            warm.step()
            torch.cuda.synchronize()
            loop.capture()
        torch.cuda.synchronize()
        spans = []
        for s in range(steps):
            stage(loop, s)
            if keep_states and mode == "graph":
                states.append(dict(plen=cache.persist_len.cpu().numpy(), kbar=cache.persist_kbar.cpu().numpy(),
                                   ring_head=int(cache.ring_head.item())))
            e0, e1 = _ev(), _ev()
            e0.record()
            if mode == "eager":
                loop.step()
            else:
                loop.replay()
            e1.record()
            spans.append((e0, e1))
            if keep_states and mode == "graph":
                torch.cuda.synchronize()
                states[-1]["topk"] = loop.topk.cpu().numpy()
        torch.cuda.synchronize()
        ms = float(np.mean([a.elapsed_time(c) for a, c in spans]))
        key = {"eager": "eager_ms_per_step", "graph": "graph_ms_per_step", "schedule": "schedule_ms_per_chunk",
               "token_graph": "token_mass_graph_ms_per_step"}[mode]
        out[key] = round(ms, 4)
        if mode == "graph":
            out["final_valid_persistent_tokens_per_head"] = float(cache.persist_len.sum(-1).float().mean())
    return out, (chunks, states, rcfg)


def cpu_baseline(cfg, heads: int, gpu_first_step: dict, rollout_record):
    """The oracle leg: the CPU oracle (as written, untuned) timed on a bounded
    sample of the decode step -- ``heads`` heads of one step (score_select,
    attend, persist_update) -- and the parity counts that only the oracle can
    give: near ties and selection mismatches of the GPU's decode-shape
    selection and update, and the cumulative selection-mismatch count of the
    rollout checked teacher-forced (every step the oracle selects from the
    GPU's pre-step state)."""
    import oracle
    import synth

    def count_topk(gpu, ora, scores, k):
        """(near-tie rows, mismatched rows, mismatches outside the near-tie band)"""
        band = mis = bad = 0
        for idx in np.ndindex(*gpu.shape[:3]):
            nt, width, boundary = oracle.near_tie_rows(scores[idx], k)
            band += nt
            a, o = set(gpu[idx].tolist()), set(ora[idx].tolist())
            if a != o:
                mis += 1
                bad += not (nt and all(abs(float(scores[idx][j]) - boundary) <= width for j in a ^ o))
        return band, mis, bad

    threads = len(os.sched_getaffinity(0))
    sub = dict(cfg, heads=heads)
    x = synth.make_step_inputs(cfg)
    xs = {k: (v[:, :heads] if v.ndim >= 3 else v) for k, v in x.items()}
    g = oracle.geometry(sub)
    t0 = time.perf_counter()
    kbar_p = oracle.pool_slots(xs["k_p"], xs["persist_len"])
    sel = oracle.score_select(xs["q"], xs["k_l"], 0, kbar_p, xs["persist_len"], g)
    oracle.attend(xs["q"], xs["k_p"], xs["v_p"], xs["persist_len"], xs["k_l"], xs["v_l"], sel["topk_idx"], g)
    state = dict(k_p=xs["k_p"], v_p=xs["v_p"], persist_len=xs["persist_len"], persist_src=xs["persist_src"],
                 persist_kbar=kbar_p)
    up = oracle.persist_update(state, sel["mass"], xs["k_l"], xs["v_l"], sel["kbar_l"], 0, 0, g)
    dt = time.perf_counter() - t0
    bl = g.block_len.astype(np.int64)
    pers = xs["persist_len"].astype(np.int64).sum(-1)
    loc = bl[sel["topk_idx"] % g.n_qblk].sum(-1)
    pairs = int((bl[None, None, :] * (pers[..., None] + loc)).sum())
    out = dict(value=4 * g.D * pairs / dt / 1e12, unit="TFLOP/s", cores=threads, kind="oracle",
               sample=f"{heads} of {cfg['heads']} heads of one decode step (score_select, attend, persist_update), "
                      f"float64 attention / float32 decisions; {dt:.1f} s",
               seconds=round(dt, 3), cpu=platform.processor() or platform.machine())
    checks = {}
    if gpu_first_step is not None and heads == cfg["heads"]:
        gd = oracle.geometry(cfg)
        nb, nm, bad = count_topk(gpu_first_step["topk"], sel["topk_idx"], sel["scores"], gd.topk)
        # update decisions implied by the GPU's new src ids (step 0: ids 0 .. n_qblk-1)
        src = gpu_first_step["after"]["persist_src"]
        keep_g = (x["persist_len"] > 0) & (src == x["persist_src"])
        heads_diff = int(sum(not np.array_equal(keep_g[i], up["keep"][i]) for i in np.ndindex(*keep_g.shape[:2])))
        checks["decode_step"] = dict(selection_rows=int(gd.B * gd.H * gd.n_qblk), near_tie_rows=nb,
                                     mismatched_rows=nm, mismatched_rows_outside_near_tie_band=bad,
                                     update_heads=int(gd.B * gd.H), update_heads_with_differences=heads_diff)
    if rollout_record is not None:
        chunks, states, rcfg = rollout_record
        gr = oracle.geometry(rcfg)
        t1 = time.perf_counter()
        rows = band = mis = bad = 0
        ring = [chunks[0]]
        for s, stt in enumerate(states):
            ring = [ring[-1], chunks[s + 1]]
            rh = stt["ring_head"]
            k_l = np.zeros((gr.B, gr.H, gr.R * gr.chunk_tokens, gr.D), np.float32)
            for logical, ch in enumerate(ring):
                c = (rh + logical) % gr.R
                k_l[:, :, c * gr.chunk_tokens:(c + 1) * gr.chunk_tokens] = ch["k"]
            ss = oracle.score_select(chunks[s + 1]["q"], k_l, rh, stt["kbar"], stt["plen"], gr)
            nb, nm, nbad = count_topk(stt["topk"], ss["topk_idx"], ss["scores"], gr.topk)
            rows += gr.B * gr.H * gr.n_qblk
            band += nb
            mis += nm
            bad += nbad
        checks["rollout_teacher_forced"] = dict(steps=len(states), selection_rows=rows, near_tie_rows=band,
                                                cumulative_selection_mismatch_rows=mis,
                                                mismatched_rows_outside_near_tie_band=bad,
                                                seconds=round(time.perf_counter() - t1, 1))
    return out, checks


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; the method shards by head with no "
                          "exchange, so --gpus N > 1 is not supported", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    import synth
    cfg = synth.workload(args.workload)
    progress(f"inputs of {args.workload}")
    b = Bench(cfg)
    torch.cuda.synchronize()
    r = time_steps(b, args.steps, args.warmup, cold_steps=args.cold_steps)
    progress(f"decode step: {r['ms']:.4f} ms")
    # the first decode step from the pristine state, for the oracle leg's counts
    b.reset()
    for name, fn in b.ops():
        fn()
        if name == "fwd":
            first_topk = b.topk.cpu().numpy()
    first = dict(topk=first_topk, after=dict(persist_len=b.live["plen"].cpu().numpy(),
                                             persist_src=b.live["psrc"].cpu().numpy()))
    p = b.p
    kern, cold, pairs = summarize(b, r, DECODE_OPS)
    flops = 4 * p.D * pairs
    value = flops / (r["ms"] * 1e-3) / 1e12
    traffic = traffic_record(args.workload).get("pbsa_fwd")
    achieved = kern["fwd"]["tflops"]
    roof = {"kernel": "pbsa_fwd", "bound": "mfma", "achieved": achieved, "peak": MI355X_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / MI355X_BF16_TFLOPS, 4),
            "traffic": round(traffic) if traffic else None}
    accs = r["acc"]
    out = {
        "metric": "PBSA decode-step ms + effective TFLOP/s (fraction of bf16 MFMA peak)",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg["dtype"], "data": "synthetic",
        "config": {"workload": f"{args.workload}: B{cfg['batch']} H{cfg['heads']} d{cfg['head_dim']} "
                               f"grid {cfg['frame_h']}x{cfg['frame_w']} "
                               f"[{cfg['block_t']},{cfg['block_h']},{cfg['block_w']}] blocks, "
                               f"{p.chunk_tokens} queries, {cfg['local_cache_size']} local + "
                               f"{cfg['persistent_cache_size']} persistent tokens, top-k ratio {cfg['topk_ratio']}",
                   "step": "ring_append + score_select + fwd + persist_update",
                   "parallelism": "single GPU"},
        "roofline": roof,
        "kernels": kern, "kernels_cold": cold,
        "step_frac_of_bf16_peak": round(value / MI355X_BF16_TFLOPS, 4),
        "pairs_per_step": pairs,
        "mean_valid_persistent_tokens": float(np.mean([a["pers_tokens"] for a in accs])),
        "mean_selected_local_tokens": float(np.mean([a["local_tokens"] for a in accs])),
        "wall_s": round(r["wall"], 3),
    }
    if not args.no_train:
        b.enable_train()
        rt = time_steps(b, args.steps, args.warmup, train=True)
        kt, _, pt = summarize(b, rt, TRAIN_OPS)
        out["train_step"] = {"step": "ring_append + score_select + fwd + bwd + persist_update",
                             "ms": round(rt["ms"], 4),
                             "tflops": round(14 * p.D * pt / (rt["ms"] * 1e-3) / 1e12, 2),
                             "bwd": kt["bwd"],
                             "bwd_frac_of_bf16_peak": round(kt["bwd"]["tflops"] / MI355X_BF16_TFLOPS, 4),
                             "bwd_traffic": (lambda t: round(t) if t else None)(
                                 traffic_record(args.workload).get("pbsa_bwd"))}
        b.grads = b.ws_b = None
        progress(f"training step: {rt['ms']:.4f} ms")
    del b
    torch.cuda.empty_cache()
    if not args.no_344:
        c344 = synth.workload("decode_344")
        b3 = Bench(c344)
        r3 = time_steps(b3, args.steps, args.warmup)
        k3, _, p3 = summarize(b3, r3, DECODE_OPS)
        out["decode_344"] = {"workload": "decode_344: the decode shape with [3,4,4] blocks (104 blocks of 48/24 "
                                         "tokens per chunk, 208 local blocks, 208 slots of 48 rows, k = 26)",
                             "ms_per_step": round(r3["ms"], 4),
                             "tflops": round(4 * b3.p.D * p3 / (r3["ms"] * 1e-3) / 1e12, 2),
                             "kernels": k3, "pairs_per_step": p3}
        del b3
        torch.cuda.empty_cache()
        progress(f"decode_344 step: {r3['ms']:.4f} ms")
    rec = None
    if args.rollout_steps > 0:
        out["rollout"], rec = run_rollout(args.rollout_steps, args.denoise_passes, keep_states=not args.no_cpu)
        progress(f"rollout: {out['rollout']}")
    if not args.no_cpu:
        progress("oracle leg")
        out["cpu_baseline"], checks = cpu_baseline(cfg, args.cpu_heads, first, rec)
        out["parity_counts"] = checks
        if "rollout_teacher_forced" in checks and "rollout" in out:
            out["rollout"]["cumulative_selection_mismatch_rows"] = \
                checks["rollout_teacher_forced"]["cumulative_selection_mismatch_rows"]
    print(json.dumps(out))


if __name__ == "__main__":
    main()
