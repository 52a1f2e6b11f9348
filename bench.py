"""Benchmark of one PBSA step at the 12-head, d=128 decode shape on one MI355X.

One step = the whole hot path over one chunk: append the chunk's K/V to the
local ring, pooled scoring + top-k selection + pooled masses, the sparse
attention forward, its backward (training), and the persistent-cache update
(which also advances the ring).  The cache state rolls from step to step, as
in a real rollout; the work of every timed step is accounted exactly by a
deterministic untimed replay that reads back the selections and slot lengths.

Prints one JSON line (see --help).  Only one GPU is supported: the method is
independent per head, so a multi-GPU run would shard heads with no exchange.
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_c1")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-accounting", action="store_true", help="skip the exact per-step FLOP replay")
    ap.add_argument("--cpu-heads", type=int, default=12, help="heads in the CPU oracle sample")
    ap.add_argument("--rollout-steps", type=int, default=80,
                    help="chunks of the graph-replayed rollout (0 skips it)")
    ap.add_argument("--cold-steps", type=int, default=5,
                    help="extra steps with a cache-evicting fill before every op (0 skips them)")
    ap.add_argument("--denoise-passes", type=int, default=4,
                    help="denoising passes per chunk in the full-schedule timing (not given by the pages)")
    return ap.parse_args()


class Bench:
    OPS = ("append", "score_select", "fwd", "bwd", "update")

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
        self.q = dev(x["q"], dt)
        # the chunk appended each step: the current chunk of the input ring
        nq = p.chunk_tokens
        self.k_new = self.pristine["k_l"][:, :, nq:2 * nq].contiguous()
        self.v_new = self.pristine["v_l"][:, :, nq:2 * nq].contiguous()
        self.dout = dev(dout, dt)
        f32 = dict(dtype=torch.float32, device="cuda")
        self.topk = torch.empty(s["topk_idx"], dtype=torch.int32, device="cuda")
        self.mass = torch.empty(s["mass"], **f32)
        self.kbar_l = torch.empty(s["kbar_local"], **f32)
        self.o = torch.empty(s["q"], dtype=dt, device="cuda")
        self.lse = torch.empty(s["lse"], **f32)
        self.dq = torch.empty(s["q"], **f32)
        self.dk_p = torch.empty(s["k_pers"], **f32)
        self.dv_p = torch.empty(s["k_pers"], **f32)
        self.dk_l = torch.empty(s["k_local"], **f32)
        self.dv_l = torch.empty(s["k_local"], **f32)
        self.n_rep = torch.empty(s["n_replaced"], dtype=torch.int32, device="cuda")
        self.ws_s = pb.workspace(p, "score_select")
        self.ws_b = pb.workspace(p, "bwd")
        self.ws_u = pb.workspace(p, "persist_update")
        self.ws_f = pb.workspace(p, "fwd")
        self.ws_fm = pb.workspace(p, "fwd_mass")
        self.tmass = torch.empty(s["mass"], **f32)
        self.step_id = 0

    def reset(self):
        for k, v in self.pristine.items():
            self.live[k].copy_(v)
        self.pkbar.copy_(self.pkbar0)
        self.step_id = 0

    def step(self, ev=None, record=None, flush=None):
        """One step.  ``ev``: per-op (start, end) event pairs to record;
        ``flush``: callable run before each op (outside its events) to evict
        the caches for cold-HBM timing."""
        pb, L, p = self.pb, self.live, self.p

        def op(i, fn):
            if flush is not None:
                flush()
            if ev is not None:
                ev[i][0].record()
            fn()
            if ev is not None:
                ev[i][1].record()

        # ring append writes into the slot the previous update freed (the
        # first step overwrites the current chunk with itself)
        op(0, lambda: pb.pbsa_ring_append(p, self.k_new, self.v_new, L["ring_head"], L["k_l"], L["v_l"]))
        op(1, lambda: pb.pbsa_score_select(p, self.q, L["k_l"], L["ring_head"], self.pkbar, L["plen"], self.topk,
                                           self.mass, self.kbar_l, self.ws_s))
        op(2, lambda: pb.pbsa_fwd(p, self.q, L["k_p"], L["v_p"], L["plen"], L["k_l"], L["v_l"], self.topk, self.o,
                                  self.lse, self.ws_f))
        op(3, lambda: pb.pbsa_bwd(p, self.q, L["k_p"], L["v_p"], L["plen"], L["k_l"], L["v_l"], self.topk, self.o,
                                  self.lse, self.dout, self.dq, self.dk_p, self.dv_p, self.dk_l, self.dv_l, self.ws_b))
        if record is not None:
            record.append(self.account())
            plen_before = L["plen"].cpu().numpy()
        op(4, lambda: pb.pbsa_persist_update(p, self.mass, L["k_l"], L["v_l"], self.kbar_l, L["ring_head"], L["step"],
                                             L["k_p"], L["v_p"], L["plen"], L["psrc"], self.pkbar, self.n_rep,
                                             self.ws_u))
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


def _events(n):
    import torch
    return [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(len(Bench.OPS))] for _ in range(n)]


def _op_stats(evs):
    """Per-op mean, median and p99 (ms) over the recorded steps."""
    out = {}
    for i, op in enumerate(Bench.OPS):
        t = np.array([e[i][0].elapsed_time(e[i][1]) for e in evs])
        out[op] = dict(mean=float(t.mean()), p50=float(np.median(t)), p99=float(np.percentile(t, 99)))
    return out


def run_gpu(args, cfg):
    import torch
    b = Bench(cfg)
    b._bl = b.block_lens().astype(np.int64)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        b.step()
    evs = _events(args.steps)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for k in range(args.steps):
        b.step(evs[k])
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    per_op = _op_stats(evs)
    # the forward with token-exact masses (the cache pass's alternative mass)
    L = b.live
    fm = []
    for k in range(args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.pb.pbsa_fwd_mass(b.p, b.q, L["k_p"], L["v_p"], L["plen"], L["k_l"], L["v_l"], b.topk, b.o, b.lse,
                           b.tmass, b.ws_fm)
        e1.record()
        fm.append((e0, e1))
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(c) for a, c in fm])
    per_op["fwd_mass"] = dict(mean=float(t.mean()), p50=float(np.median(t)), p99=float(np.percentile(t, 99)))
    # cold-cache pass: a 1 GiB fill before every op evicts L2 and the MALL
    cold = None
    if args.cold_steps > 0:
        junk = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        cevs = _events(args.cold_steps)
        for k in range(args.cold_steps):
            b.step(cevs[k], flush=lambda: junk.fill_(k & 0xFF))
        torch.cuda.synchronize()
        cold = _op_stats(cevs)
        del junk
    # exact accounting by deterministic replay
    acc = None
    if not args.no_accounting:
        b.reset()
        for _ in range(args.warmup):
            b.step()
        rec = []
        for _ in range(args.steps):
            b.step(record=rec)
        torch.cuda.synchronize()
        acc = rec
    return b, total_ms, wall, per_op, cold, acc


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


def run_rollout(cfg, steps: int, denoise: int):
    """Long rollout: chunk s's q/k/v (seeded, drifting planted blocks) are staged
    into the loop's buffers (device-to-device) and one captured graph runs the
    cache pass (ring append, score/select, fwd, persistent update).  Also times
    the per-chunk schedule with `denoise` denoising passes before the cache pass."""
    import torch
    import block_sparse_attention_15_amd as pb
    from block_sparse_attention_15_amd.rollout import DecodeLoop
    import synth
    rcfg = synth.workload("rollout_c4", steps=steps)
    stream = synth.RolloutStream(rcfg)
    x = synth.make_step_inputs(rcfg)
    p = pb.pbsa_plan(rcfg)
    dt = p.torch_dtype
    dev = lambda a: torch.from_numpy(a).to(dt).cuda()
    chunks = [stream.chunk(s) for s in range(-1, steps)]
    dq = torch.stack([dev(c["q"]) for c in chunks[1:]])
    dk = torch.stack([dev(c["k"]) for c in chunks[1:]])
    dv = torch.stack([dev(c["v"]) for c in chunks[1:]])

    def fresh(mass="pooled"):
        cache = pb.PBSACache(p)
        cache.k_pers.copy_(dev(x["k_p"]))
        cache.v_pers.copy_(dev(x["v_p"]))
        cache.persist_len.copy_(torch.from_numpy(x["persist_len"]).cuda())
        cache.persist_src.copy_(torch.from_numpy(x["persist_src"]).cuda())
        ct = p.chunk_tokens
        cache.k_local[:, :, :ct].copy_(dev(chunks[0]["k"]))
        cache.v_local[:, :, :ct].copy_(dev(chunks[0]["v"]))
        cache.refresh_pooled_keys()
        return cache, DecodeLoop(p, cache, mass=mass)

    out = {"steps": steps, "denoise_passes": denoise}
    for mode in ("eager", "graph", "schedule", "token_graph"):
        mass = "token" if mode == "token_graph" else "pooled"
        cache, loop = fresh(mass)
        nd = denoise if mode == "schedule" else 0
        loop.load_chunk(dq[0], dk[0], dv[0])
        if mode != "eager":
            _, warm = fresh(mass)
            warm.load_chunk(dq[0], dk[0], dv[0])
            warm.step(nd)
            torch.cuda.synchronize()
            loop.capture(nd)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for s in range(steps):
            loop.load_chunk(dq[s], dk[s], dv[s])
            if mode == "eager":
                loop.step(0)
            else:
                loop.replay()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        if mode == "eager":
            out["eager_ms_per_step"] = round(ms, 4)
        elif mode == "graph":
            out["graph_ms_per_step"] = round(ms, 4)
            out["final_valid_persistent_tokens_per_head"] = float(cache.persist_len.sum(-1).float().mean())
        elif mode == "schedule":
            out["schedule_ms_per_chunk"] = round(ms, 4)
        else:
            out["token_mass_graph_ms_per_step"] = round(ms, 4)
    return out


def cpu_baseline(cfg, heads: int):
    """The oracle (as written, untuned) on a bounded sample: `heads` heads of the step."""
    import oracle
    import synth
    threads = len(os.sched_getaffinity(0))
    sub = dict(cfg, heads=heads)
    x = synth.make_step_inputs(cfg)
    xs = {k: (v[:, :heads] if v.ndim >= 3 else v) for k, v in x.items()}
    dout = synth.make_dout(dict(cfg, dout_seed=3))[:, :heads]
    g = oracle.geometry(sub)
    t0 = time.perf_counter()
    kbar_p = oracle.pool_slots(xs["k_p"], xs["persist_len"])
    sel = oracle.score_select(xs["q"], xs["k_l"], 0, kbar_p, xs["persist_len"], g)
    O, L = oracle.attend(xs["q"], xs["k_p"], xs["v_p"], xs["persist_len"], xs["k_l"], xs["v_l"],
                         sel["topk_idx"], g)
    oracle.attend_bwd(xs["q"], xs["k_p"], xs["v_p"], xs["persist_len"], xs["k_l"], xs["v_l"], sel["topk_idx"],
                      dout, g)
    state = dict(k_p=xs["k_p"], v_p=xs["v_p"], persist_len=xs["persist_len"], persist_src=xs["persist_src"],
                 persist_kbar=kbar_p)
    oracle.persist_update(state, sel["mass"], xs["k_l"], xs["v_l"], sel["kbar_l"], 0, 0, g)
    dt = time.perf_counter() - t0
    bl = g.block_len.astype(np.int64)
    pers = xs["persist_len"].astype(np.int64).sum(-1)
    loc = bl[sel["topk_idx"] % g.n_qblk].sum(-1)
    pairs = int((bl[None, None, :] * (pers[..., None] + loc)).sum())
    flops = 14 * g.D * pairs
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=threads, kind="oracle",
                sample=f"{heads} of {cfg['heads']} heads of one step (score_select, attend, attend_bwd, "
                       f"persist_update), float64 attention / float32 decisions; {dt:.1f} s",
                seconds=dt, cpu=platform.processor() or platform.machine())


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; the method shards by head with no "
                          "exchange, so --gpus N > 1 is not supported", "n_gpus": args.gpus}))
        sys.exit(2)
    import synth
    cfg = synth.workload(args.workload)
    b, total_ms, wall, stats, cold, acc = run_gpu(args, cfg)
    p = b.p
    ms_step = total_ms / args.steps
    out = {"metric": "PBSA decode-step ms + effective TFLOP/s (fraction of bf16 MFMA peak)"}
    per_op = {op: v["mean"] for op, v in stats.items()}
    kern = {op: {"ms": round(v["mean"], 4), "p50_ms": round(v["p50"], 4), "p99_ms": round(v["p99"], 4)}
            for op, v in stats.items()}
    kern["fwd_mass"]["extra_ms_over_fwd"] = round(per_op["fwd_mass"] - per_op["fwd"], 4)
    kern_cold = {}
    if acc:
        pairs = float(np.mean([a["pairs"] for a in acc]))
        fwd_flops = 4 * p.D * pairs
        bwd_flops = 10 * p.D * pairs
        step_tflops = (fwd_flops + bwd_flops) / (ms_step * 1e-3) / 1e12
        kern["fwd"].update(tflops=round(fwd_flops / (per_op["fwd"] * 1e-3) / 1e12, 2), gflop=round(fwd_flops / 1e9, 2))
        kern["bwd"].update(tflops=round(bwd_flops / (per_op["bwd"] * 1e-3) / 1e12, 2), gflop=round(bwd_flops / 1e9, 2))
        B, H, D, esz = p.B, p.H, p.D, (2 if cfg["dtype"] == "bf16" else 4)
        score_bytes = B * H * (p.chunk_tokens + p.local_tokens) * D * esz + B * H * p.persistent_slots * D * 4
        kern["score_select"].update(gbs=round(score_bytes / (per_op["score_select"] * 1e-3) / 1e9, 1),
                                    mb=round(score_bytes / 1e6, 2))
        ub = float(np.mean([a["update_bytes"] for a in acc]))
        kern["update"].update(gbs=round(ub / (per_op["update"] * 1e-3) / 1e9, 1), mb=round(ub / 1e6, 2))
        app = 2 * 2 * B * H * p.chunk_tokens * D * esz
        kern["append"].update(gbs=round(app / (per_op["append"] * 1e-3) / 1e9, 1), mb=round(app / 1e6, 2))
        if cold:
            hbm = dict(append=app, score_select=score_bytes, update=ub)
            for op in Bench.OPS:
                c = {"ms": round(cold[op]["mean"], 4), "p50_ms": round(cold[op]["p50"], 4)}
                if op in hbm:
                    c["gbs"] = round(hbm[op] / (cold[op]["mean"] * 1e-3) / 1e9, 1)
                    c["frac_hbm"] = round(c["gbs"] / MI355X_HBM_GBS, 4)
                kern_cold[op] = c
        dom = max(("fwd", "bwd"), key=lambda k: per_op[k])
        achieved = kern[dom]["tflops"]
        traffic = traffic_record(args.workload).get(f"pbsa_{dom}")
        roof = {"kernel": f"pbsa_{dom}", "bound": "mfma", "achieved": achieved, "peak": MI355X_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MI355X_BF16_TFLOPS, 4),
                "traffic": round(traffic) if traffic else None}
        value = step_tflops
        extra = dict(pairs_per_step=pairs, mean_valid_persistent_tokens=float(np.mean([a["pers_tokens"] for a in acc])),
                     mean_selected_local_tokens=float(np.mean([a["local_tokens"] for a in acc])))
    else:
        value, roof, extra = None, None, {}
    decode_ms = per_op["append"] + per_op["score_select"] + per_op["fwd"] + per_op["update"]
    decode_p50 = sum(stats[op]["p50"] for op in ("append", "score_select", "fwd", "update"))
    out.update({
        "value": round(value, 3) if value else None, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "decode_step_ms": round(decode_ms, 4),
        "decode_step_p50_ms": round(decode_p50, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg["dtype"],
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: B{cfg['batch']} H{cfg['heads']} d{cfg['head_dim']} "
                               f"grid {cfg['frame_h']}x{cfg['frame_w']} "
                               f"[{cfg['block_t']},{cfg['block_h']},{cfg['block_w']}] blocks, "
                               f"{p.chunk_tokens} queries, {cfg['local_cache_size']} local + "
                               f"{cfg['persistent_cache_size']} persistent tokens, top-k ratio {cfg['topk_ratio']}",
                   "step": "ring_append + score_select + fwd + bwd + persist_update",
                   "parallelism": "single GPU"},
        "kernels": kern, "kernels_cold": kern_cold or None, "roofline": roof, "wall_s": round(wall, 3), **extra,
    })
    if args.rollout_steps > 0:
        out["rollout"] = run_rollout(cfg, args.rollout_steps, args.denoise_passes)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_heads)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
