"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Tolerances: fp32 inputs, 1e-5 absolute on O, 1e-4 on gradients.  bf16
inputs (P rounded to bf16 before P.V, O stored as bf16): max-abs error 1e-2 on
O and gradients (unit-variance V), plus a relative-L2 bound of 1e-2 (O) and
2e-2 (gradients) since the max-abs gate alone is loose at these magnitudes
(std(O) ~ 0.02).  Selections are bit-exact except counted near ties (oracle
score gap below 1e-4 of the row's score spread); persistent state is
bit-exact given the decisions.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import block_sparse_attention_15_amd as pb
from pbsa_harness import (GpuStep, compare_topk, compare_update_decisions, decisions_from_state, dev, host,
                          rel_l2)

pytestmark = pytest.mark.gpu


def ragged(**kw):
    """14x22 grid: blocks of 64, 64, 48, 48, 48, 36 tokens; 2-frame chunks, R=2."""
    c = dict(batch=1, heads=2, head_dim=128, frame_h=14, frame_w=22, block_t=1, block_h=8, block_w=8,
             chunk_frames=2, total_cache_size=4 * 308 + 3 * 308, local_cache_size=4 * 308,
             persistent_cache_size=3 * 308, use_local_block_sparse_attn=1, topk_ratio=0.25, softmax_scale=0.0,
             dtype="bf16", seed=21, plant_frac=0.1, alpha=4.0)
    c.update(kw)
    return c


SMALL = {
    "tiny_fp32": synth.workload("tiny_fp32"),
    "ragged_bf16": ragged(),
    "ragged_bf16_d64_b2": ragged(head_dim=64, batch=2, seed=22),
    "ragged_fp32": ragged(dtype="fp32", seed=23),
    "dense_local_bf16": ragged(use_local_block_sparse_attn=0, seed=24),
    # dense local window of 36 blocks (K = 36): 9 KB row tables in the local kernels (three
    # workgroups per CU instead of four)
    "dense_local_wide_bf16": ragged(use_local_block_sparse_attn=0, local_cache_size=6 * 308,
                                    total_cache_size=6 * 308 + 3 * 308, seed=26),
    # dense local window of 516 blocks (K = 516): more selected blocks than the local kernels'
    # LDS row tables hold at head_dim 128, so their gathers look the row tokens up in global memory
    "dense_local_huge_bf16": ragged(use_local_block_sparse_attn=0, local_cache_size=86 * 308,
                                    total_cache_size=86 * 308 + 3 * 308, seed=29),
    # [3,4,4] blocks on a 10x14 grid: 12 blocks per 3-frame group (48/24/24/12 tokens)
    "block344_bf16": ragged(frame_h=10, frame_w=14, block_t=3, block_h=4, block_w=4, chunk_frames=3,
                            total_cache_size=9 * 140, local_cache_size=6 * 140, persistent_cache_size=3 * 140,
                            seed=25),
    # the same [3,4,4] blocks at head_dim 64, two batch entries: 48-row slots on the packed
    # persistent dV pass and the packed dK grid at the smaller head size
    "block344_bf16_d64_b2": ragged(frame_h=10, frame_w=14, block_t=3, block_h=4, block_w=4, chunk_frames=3,
                                   total_cache_size=9 * 140, local_cache_size=6 * 140,
                                   persistent_cache_size=3 * 140, head_dim=64, batch=2, seed=27),
    # no persistent memory: plain local block-sparse attention; the update only advances the ring
    "no_persistent_bf16": ragged(persistent_cache_size=0, total_cache_size=4 * 308, seed=51),
    # 16x16 grid, head_dim 64, 8 slots: a slot count that is not a multiple of the persistent
    # kernels' three-deep load rotation
    "tiny_bf16": {**synth.workload("tiny_fp32"), "dtype": "bf16", "seed": 61},
    # 252 persistent slots: the row tables of the packed persistent kernels (forward and dQ/dK)
    # would exceed their 60 KB of LDS, so the per-slot kernels run, with the stored dS tiles
    "big_persistent_bf16": ragged(persistent_cache_size=42 * 308, total_cache_size=4 * 308 + 42 * 308, seed=28),
    # 8x8 grid, one block per frame: 64-query chunks (two query tiles), one persistent slot,
    # two local blocks, top-1 -- most of a workgroup's slots and steps are padding
    "micro_bf16": ragged(frame_h=8, frame_w=8, chunk_frames=1, total_cache_size=3 * 64, local_cache_size=2 * 64,
                         persistent_cache_size=64, topk_ratio=0.5, seed=71),
}


def tol(cfg):
    if cfg["dtype"] == "fp32":
        return dict(o_abs=1e-5, o_rel=1e-5, lse=1e-5, g_abs=1e-4, g_rel=1e-4)
    return dict(o_abs=1e-2, o_rel=1e-2, lse=2e-3, g_abs=1e-2, g_rel=2e-2)


def oracle_select(cfg, x, ring_head):
    g = oracle.geometry(cfg)
    kbar_p = oracle.pool_slots(x["k_p"], x["persist_len"])
    return g, kbar_p, oracle.score_select(x["q"], x["k_l"], ring_head, kbar_p, x["persist_len"], g)


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("ring_head", [0, 1])
def test_score_select(name, ring_head):
    cfg = SMALL[name]
    x = synth.make_step_inputs(cfg)
    x["ring_head"][:] = ring_head
    g, kbar_p, sel = oracle_select(cfg, x, ring_head)
    st = GpuStep(cfg, x)
    st.score_select()
    torch.cuda.synchronize()
    np.testing.assert_allclose(host(st.pkbar), kbar_p, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(host(st.kbar_l), sel["kbar_l"], rtol=1e-5, atol=1e-6)
    nb, nm = compare_topk(host(st.topk), sel["topk_idx"], sel["scores"], g.topk)
    print(f"{name}: near-tie rows {nb}, mismatched rows {nm}")
    np.testing.assert_allclose(host(st.mass), sel["mass"], rtol=1e-4, atol=1e-5)


@pytest.mark.parametrize("name", list(SMALL))
def test_fwd(name):
    cfg = SMALL[name]
    x = synth.make_step_inputs(cfg)
    g, _, sel = oracle_select(cfg, x, 0)
    O, L = oracle.attend(x["q"], x["k_p"], x["v_p"], x["persist_len"], x["k_l"], x["v_l"], sel["topk_idx"], g)
    st = GpuStep(cfg, x)
    st.fwd(dev(sel["topk_idx"]))
    torch.cuda.synchronize()
    t = tol(cfg)
    o = host(st.o)
    err = np.abs(o - O).max()
    print(f"{name}: O max-abs {err:.3g} rel-L2 {rel_l2(o, O):.3g}")
    assert err <= t["o_abs"] and rel_l2(o, O) <= t["o_rel"]
    np.testing.assert_allclose(host(st.lse), L, rtol=0, atol=t["lse"])


@pytest.mark.parametrize("name", list(SMALL))
def test_bwd(name):
    cfg = SMALL[name]
    x = synth.make_step_inputs(cfg)
    g, _, sel = oracle_select(cfg, x, 0)
    dout = synth.make_dout(cfg, seed=cfg["seed"] + 100)
    ref = oracle.attend_bwd(x["q"], x["k_p"], x["v_p"], x["persist_len"], x["k_l"], x["v_l"], sel["topk_idx"],
                            dout, g)
    st = GpuStep(cfg, x)
    idx = dev(sel["topk_idx"])
    st.fwd(idx)
    gr = st.bwd(dev(dout, st.p.torch_dtype), idx)
    torch.cuda.synchronize()
    t = tol(cfg)
    for k in ("dq", "dk_p", "dv_p", "dk_l", "dv_l"):
        a = host(gr[k])
        if a.size == 0:      # no persistent slots
            continue
        assert np.isfinite(a).all(), k
        err = np.abs(a - ref[k]).max()
        r = rel_l2(a, ref[k])
        print(f"{name}: {k} max-abs {err:.3g} rel-L2 {r:.3g}")
        assert err <= t["g_abs"] and r <= t["g_rel"], k


@pytest.mark.parametrize("name", ["ragged_bf16", "block344_bf16", "tiny_bf16"])
def test_fwd_bwd_empty_slots(name):
    """Empty persistent slots (length 0) beside full and partial ones.  The
    emptied slots keep their K/V rows, which must be ignored; their gradient
    rows must come back zero."""
    cfg = SMALL[name]
    x = synth.make_step_inputs(cfg)
    S = x["persist_len"].shape[-1]
    empty = [s for s in (1, 4, 9) if s < S]
    x["persist_len"][..., empty] = 0
    g, _, sel = oracle_select(cfg, x, 0)
    O, L = oracle.attend(x["q"], x["k_p"], x["v_p"], x["persist_len"], x["k_l"], x["v_l"], sel["topk_idx"], g)
    dout = synth.make_dout(cfg, seed=cfg["seed"] + 100)
    ref = oracle.attend_bwd(x["q"], x["k_p"], x["v_p"], x["persist_len"], x["k_l"], x["v_l"], sel["topk_idx"],
                            dout, g)
    st = GpuStep(cfg, x)
    idx = dev(sel["topk_idx"])
    st.fwd(idx)
    gr = st.bwd(dev(dout, st.p.torch_dtype), idx)
    torch.cuda.synchronize()
    t = tol(cfg)
    o = host(st.o)
    err = np.abs(o - O).max()
    print(f"{name}: empty slots {empty}: O max-abs {err:.3g} rel-L2 {rel_l2(o, O):.3g}")
    assert err <= t["o_abs"] and rel_l2(o, O) <= t["o_rel"]
    np.testing.assert_allclose(host(st.lse), L, rtol=0, atol=t["lse"])
    for k in ("dq", "dk_p", "dv_p", "dk_l", "dv_l"):
        a = host(gr[k])
        assert np.isfinite(a).all(), k
        err = np.abs(a - ref[k]).max()
        r = rel_l2(a, ref[k])
        print(f"{name}: {k} max-abs {err:.3g} rel-L2 {r:.3g}")
        assert err <= t["g_abs"] and r <= t["g_rel"], k
    for k in ("dk_p", "dv_p"):
        assert not host(gr[k])[..., empty, :, :].any(), f"{k}: empty slots must get zero gradient"


@pytest.mark.parametrize("name", ["ragged_bf16", "ragged_bf16_d64_b2", "block344_bf16", "tiny_bf16"])
def test_bwd_recompute_path(name):
    """With the persistent dS tiles switched off (bwd_ds_max_mb = -1) the
    backward's dK pass recomputes dS instead of reading it from the
    workspace: the same gradients from a smaller workspace."""
    stored = pb.pbsa_plan(SMALL[name]).ws_bwd
    cfg = dict(SMALL[name], bwd_ds_max_mb=-1)
    assert pb.pbsa_plan(cfg).ws_bwd < stored
    x = synth.make_step_inputs(cfg)
    x["persist_len"][..., 1] = 0
    x["persist_len"][..., 2] = min(x["k_p"].shape[-2], 40)
    g, _, sel = oracle_select(cfg, x, 0)
    dout = synth.make_dout(cfg, seed=cfg["seed"] + 300)
    ref = oracle.attend_bwd(x["q"], x["k_p"], x["v_p"], x["persist_len"], x["k_l"], x["v_l"], sel["topk_idx"],
                            dout, g)
    st = GpuStep(cfg, x)
    idx = dev(sel["topk_idx"])
    st.fwd(idx)
    gr = st.bwd(dev(dout, st.p.torch_dtype), idx)
    torch.cuda.synchronize()
    t = tol(cfg)
    for k in ("dq", "dk_p", "dv_p", "dk_l", "dv_l"):
        a = host(gr[k])
        assert np.isfinite(a).all(), k
        err = np.abs(a - ref[k]).max()
        r = rel_l2(a, ref[k])
        print(f"{name} (recomputed dS): {k} max-abs {err:.3g} rel-L2 {r:.3g}")
        assert err <= t["g_abs"] and r <= t["g_rel"], k


@pytest.mark.parametrize("name", ["ragged_bf16", "block344_bf16"])
def test_bwd_very_negative_scores(name):
    """Every score near -120 (queries and keys shifted in opposite directions),
    beside partial persistent slots and short local blocks.  The dQ kernels
    take no key mask: key rows that do not exist are zero, and exp(-lse) of
    such a row (about e^120, beyond fp32) must be clamped, not overflow into
    inf * 0 = NaN."""
    cfg = SMALL[name]
    x = synth.make_step_inputs(cfg)
    C = x["k_p"].shape[-2]
    S = x["persist_len"].shape[-1]
    x["persist_len"][..., 0] = min(C, 17)
    if S > 3:
        x["persist_len"][..., 3] = min(C, 40)
    D = x["q"].shape[-1]
    scale = cfg.get("softmax_scale") or D ** -0.5
    shift = np.float32(np.sqrt(120.0 / scale / D))  # scale * (-shift^2 * D) = -120
    x["q"] = synth.bf16_round(x["q"] - shift)
    for k in ("k_p", "k_l"):
        x[k] = synth.bf16_round(x[k] + shift)
    g, _, sel = oracle_select(cfg, x, 0)
    O, L = oracle.attend(x["q"], x["k_p"], x["v_p"], x["persist_len"], x["k_l"], x["v_l"], sel["topk_idx"], g)
    assert L.max() < -80, "scores are not as negative as intended"
    dout = synth.make_dout(cfg, seed=cfg["seed"] + 200)
    ref = oracle.attend_bwd(x["q"], x["k_p"], x["v_p"], x["persist_len"], x["k_l"], x["v_l"], sel["topk_idx"],
                            dout, g)
    st = GpuStep(cfg, x)
    idx = dev(sel["topk_idx"])
    st.fwd(idx)
    gr = st.bwd(dev(dout, st.p.torch_dtype), idx)
    torch.cuda.synchronize()
    t = tol(cfg)
    for k in ("dq", "dk_p", "dv_p", "dk_l", "dv_l"):
        a = host(gr[k])
        assert np.isfinite(a).all(), k
        scale = max(1.0, float(np.abs(ref[k]).max()))
        err = np.abs(a - ref[k]).max()
        r = rel_l2(a, ref[k])
        print(f"{name}: {k} max-abs {err:.3g} (of {scale:.3g}) rel-L2 {r:.3g}")
        assert err <= t["g_abs"] * scale and r <= t["g_rel"], k


# shapes for the update only: 600 persistent slots and 12 entrants, 612
# candidates, the decision's 16-keys-per-lane tier (SMALL and the decode
# shapes take the 4- and 8-key tiers, the size-limit test the 64-key one)
UPDATE_EXTRA = {
    "huge_persistent_bf16": ragged(persistent_cache_size=100 * 308, total_cache_size=4 * 308 + 100 * 308, seed=31),
}


@pytest.mark.parametrize("name", list(SMALL) + list(UPDATE_EXTRA))
@pytest.mark.parametrize("ring_head", [0, 1])
def test_update(name, ring_head):
    cfg = SMALL[name] if name in SMALL else UPDATE_EXTRA[name]
    x = synth.make_step_inputs(cfg)
    x["ring_head"][:] = ring_head
    if name == "ragged_bf16":
        x["persist_len"][..., ::5] = 0           # some empty slots
        x["k_p"][..., ::5, :, :] = 0
        x["v_p"][..., ::5, :, :] = 0
    g, kbar_p, sel = oracle_select(cfg, x, ring_head)
    step_id = 3
    before = dict(k_p=x["k_p"], v_p=x["v_p"], persist_len=x["persist_len"], persist_src=x["persist_src"],
                  persist_kbar=kbar_p)
    ref = oracle.persist_update(before, sel["mass"], x["k_l"], x["v_l"], sel["kbar_l"], ring_head, step_id, g)

    # (1) the whole GPU path: its own masses and decisions
    st = GpuStep(cfg, x)
    st.score_select()
    st.update(step_id)
    torch.cuda.synchronize()
    after = st.state()
    assert after["ring_head"] == (ring_head + 1) % g.R
    keep_g, admit_g = decisions_from_state(before, after, step_id, g.n_qblk)
    nd = compare_update_decisions(keep_g, admit_g, ref["keep"], ref["admit"], sel["mass"], x["persist_len"],
                                  ring_head, g)
    print(f"{name}: heads with near-tie decision differences: {nd}")
    # data movement with the GPU's decisions must be bit-exact
    gpu_kbar_l = host(st.kbar_l)
    before_g = dict(before, persist_kbar=host(GpuStep(cfg, x).pkbar))
    moved = oracle.apply_update(before_g, keep_g, admit_g, x["k_l"], x["v_l"], gpu_kbar_l, ring_head, step_id, g)
    for k in ("k_p", "v_p", "persist_len", "persist_src"):
        np.testing.assert_array_equal(after[k], moved[k], err_msg=k)
    np.testing.assert_array_equal(after["persist_kbar"], moved["persist_kbar"])
    np.testing.assert_array_equal(host(st.n_rep), admit_g.sum(-1))

    # (2) pure data movement: oracle masses in, oracle state out, no exemption
    st2 = GpuStep(cfg, x)
    st2.score_select()
    st2.update(step_id, mass=dev(sel["mass"]))
    torch.cuda.synchronize()
    a2 = st2.state()
    for k in ("k_p", "v_p", "persist_len", "persist_src"):
        np.testing.assert_array_equal(a2[k], ref[k], err_msg=k)
    np.testing.assert_allclose(a2["persist_kbar"], ref["persist_kbar"], rtol=1e-5, atol=1e-6)
    np.testing.assert_array_equal(host(st2.n_rep), ref["n_replaced"])


def test_ring_append_and_empty_cache_fill():
    cfg = SMALL["ragged_bf16"]
    x = synth.make_step_inputs(cfg)
    g = oracle.geometry(cfg)
    st = GpuStep(cfg, x)
    st.ring_head.fill_(1)
    kn = torch.randn(st.q.shape, device="cuda").to(st.q.dtype)
    vn = torch.randn(st.q.shape, device="cuda").to(st.q.dtype)
    import block_sparse_attention_15_amd as pb
    kbar_before = st.kbar_l.clone()
    pb.pbsa_ring_append(st.p, kn, vn, st.ring_head, st.k_l, st.v_l, st.kbar_l)
    torch.cuda.synchronize()
    slot = (1 + g.R - 1) % g.R
    # the appended chunk's pooled keys, and only those, are rewritten
    k_ref = x["k_l"].copy()
    k_ref[:, :, slot * g.chunk_tokens:(slot + 1) * g.chunk_tokens] = host(kn)
    want = oracle.pool_local_blocks(k_ref, g)
    got = host(st.kbar_l)
    rows = slice(slot * g.n_qblk, (slot + 1) * g.n_qblk)
    np.testing.assert_allclose(got[:, :, rows], want[:, :, rows], rtol=1e-5, atol=1e-6)
    keep = np.ones(g.n_lblk, bool)
    keep[rows] = False
    np.testing.assert_array_equal(got[:, :, keep], host(kbar_before)[:, :, keep])
    assert torch.equal(st.k_l[:, :, slot * g.chunk_tokens:(slot + 1) * g.chunk_tokens], kn)
    assert torch.equal(st.v_l[:, :, slot * g.chunk_tokens:(slot + 1) * g.chunk_tokens], vn)
    other = 1 - slot
    np.testing.assert_array_equal(host(st.k_l[:, :, other * g.chunk_tokens:(other + 1) * g.chunk_tokens]),
                                  x["k_l"][:, :, other * g.chunk_tokens:(other + 1) * g.chunk_tokens])


# ---------------------------------------------------------------------------
# the 12-head, d=128, 4680-query decode step at full size
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def c1():
    cfg = synth.workload("decode_c1")
    x = synth.make_step_inputs(cfg)
    g, kbar_p, sel = oracle_select(cfg, x, 0)
    return cfg, x, g, kbar_p, sel


def test_c1_score_select(c1):
    cfg, x, g, kbar_p, sel = c1
    st = GpuStep(cfg, x)
    st.score_select()
    torch.cuda.synchronize()
    nb, nm = compare_topk(host(st.topk), sel["topk_idx"], sel["scores"], g.topk)
    print(f"decode_c1: near-tie rows {nb} of {g.B * g.H * g.n_qblk}, mismatched rows {nm}")
    np.testing.assert_allclose(host(st.mass), sel["mass"], rtol=1e-4, atol=1e-5)
    np.testing.assert_allclose(host(st.kbar_l), sel["kbar_l"], rtol=1e-5, atol=1e-6)


def test_c1_fwd_all_blocks(c1):
    """O and LSE of every query block of every head at the decode shape."""
    cfg, x, g, kbar_p, sel = c1
    st = GpuStep(cfg, x)
    st.fwd(dev(sel["topk_idx"]))
    torch.cuda.synchronize()
    O, L = oracle.attend(x["q"], x["k_p"], x["v_p"], x["persist_len"], x["k_l"], x["v_l"], sel["topk_idx"], g)
    o = host(st.o)
    err = np.abs(o - O).max()
    r = rel_l2(o, O)
    worst = max(rel_l2(o[0, h], O[0, h]) for h in range(g.H))
    print(f"decode_c1 fwd, all {g.H} heads x {g.n_qblk} query blocks: O max-abs {err:.3g} rel-L2 {r:.3g} "
          f"(worst head {worst:.3g})")
    assert err <= 1e-2 and r <= 1e-2 and worst <= 1e-2
    np.testing.assert_allclose(host(st.lse), L, atol=2e-3)


def test_c1_update(c1):
    cfg, x, g, kbar_p, sel = c1
    step_id = 5
    before = dict(k_p=x["k_p"], v_p=x["v_p"], persist_len=x["persist_len"], persist_src=x["persist_src"],
                  persist_kbar=kbar_p)
    ref = oracle.persist_update(before, sel["mass"], x["k_l"], x["v_l"], sel["kbar_l"], 0, step_id, g)
    st = GpuStep(cfg, x)
    st.score_select()
    st.update(step_id)
    torch.cuda.synchronize()
    after = st.state()
    keep_g, admit_g = decisions_from_state(before, after, step_id, g.n_qblk)
    nd = compare_update_decisions(keep_g, admit_g, ref["keep"], ref["admit"], sel["mass"], x["persist_len"], 0, g)
    print(f"decode_c1 update: replaced per head {host(st.n_rep).tolist()}, near-tie heads {nd}")
    moved = oracle.apply_update(dict(before, persist_kbar=host(GpuStep(cfg, x).pkbar)), keep_g, admit_g,
                                x["k_l"], x["v_l"], host(st.kbar_l), 0, step_id, g)
    for k in ("k_p", "v_p", "persist_len", "persist_src", "persist_kbar"):
        np.testing.assert_array_equal(after[k], moved[k], err_msg=k)
    st2 = GpuStep(cfg, x)
    st2.score_select()
    st2.update(step_id, mass=dev(sel["mass"]))
    torch.cuda.synchronize()
    a2 = st2.state()
    for k in ("k_p", "v_p", "persist_len", "persist_src"):
        np.testing.assert_array_equal(a2[k], ref[k], err_msg=k)


@pytest.fixture(scope="module")
def c3_ref(c1):
    cfg, x, g, kbar_p, sel = c1
    dout = synth.make_dout(synth.workload("backward_c3"))
    ref = oracle.attend_bwd(x["q"], x["k_p"], x["v_p"], x["persist_len"], x["k_l"], x["v_l"], sel["topk_idx"],
                            dout, g)
    return dout, ref


def test_c3_bwd_all_heads(c1, c3_ref):
    """All five gradients of every head, element by element, at the decode
    shape (stored-dS path), plus the sum identities as extra checks."""
    cfg, x, g, kbar_p, sel = c1
    dout, ref = c3_ref
    st = GpuStep(cfg, x)
    idx = dev(sel["topk_idx"])
    st.fwd(idx)
    gr = st.bwd(dev(dout, torch.bfloat16), idx)
    torch.cuda.synchronize()
    for k in ("dq", "dk_p", "dv_p", "dk_l", "dv_l"):
        a = host(gr[k])
        assert np.isfinite(a).all(), k
        err = np.abs(a - ref[k]).max()
        r = rel_l2(a, ref[k])
        worst = max(rel_l2(a[0, h], ref[k][0, h]) for h in range(g.H))
        print(f"decode_c1 bwd, all heads: {k} max-abs {err:.3g} rel-L2 {r:.3g} (worst head {worst:.3g})")
        assert err <= 1e-2 and r <= 2e-2 and worst <= 2e-2, k
    for h in range(g.H):
        dk = np.concatenate([host(gr["dk_p"])[0, h].reshape(-1, g.D), host(gr["dk_l"])[0, h].reshape(-1, g.D)])
        dv = np.concatenate([host(gr["dv_p"])[0, h].reshape(-1, g.D), host(gr["dv_l"])[0, h].reshape(-1, g.D)])
        dk, dv = dk.astype(np.float64), dv.astype(np.float64)
        assert np.abs(dk.sum(0)).max() <= 1e-3 * np.abs(dk).sum(0).max(), h
        want = dout[0, h].astype(np.float64).reshape(-1, g.D).sum(0)
        assert np.abs(dv.sum(0) - want).max() <= 1e-2 * np.abs(want).max() + 1e-2, h


def test_c1_determinism(c1):
    cfg, x, g, kbar_p, sel = c1
    st = GpuStep(cfg, x)
    st.score_select()
    st.fwd()
    torch.cuda.synchronize()
    o1, l1, t1, m1 = st.o.clone(), st.lse.clone(), st.topk.clone(), st.mass.clone()
    dout = dev(synth.make_dout(synth.workload("backward_c3")), torch.bfloat16)
    g1 = st.bwd(dout)
    st.score_select()
    st.fwd()
    g2 = st.bwd(dout)
    torch.cuda.synchronize()
    assert torch.equal(t1, st.topk) and torch.equal(m1, st.mass)
    assert torch.equal(o1, st.o) and torch.equal(l1, st.lse)
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k


# ---------------------------------------------------------------------------
# [3,4,4] blocks at the decode shape (104 blocks per chunk, 48-row slots)
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def c344():
    cfg = synth.workload("decode_c1", block_t=3, block_h=4, block_w=4, seed=6)
    x = synth.make_step_inputs(cfg)
    g, kbar_p, sel = oracle_select(cfg, x, 0)
    return cfg, x, g, kbar_p, sel


def test_c344_score_select_fwd_update(c344):
    cfg, x, g, kbar_p, sel = c344
    st = GpuStep(cfg, x)
    st.score_select()
    torch.cuda.synchronize()
    nb, nm = compare_topk(host(st.topk), sel["topk_idx"], sel["scores"], g.topk)
    print(f"[3,4,4] decode shape: near-tie rows {nb}, mismatched rows {nm}")
    np.testing.assert_allclose(host(st.mass), sel["mass"], rtol=1e-4, atol=1e-5)
    st.fwd(dev(sel["topk_idx"]))
    torch.cuda.synchronize()
    O, L = oracle.attend(x["q"], x["k_p"], x["v_p"], x["persist_len"], x["k_l"], x["v_l"], sel["topk_idx"], g)
    o = host(st.o)
    print(f"[3,4,4] decode shape fwd, all heads and blocks: O max-abs {np.abs(o - O).max():.3g} "
          f"rel-L2 {rel_l2(o, O):.3g}")
    assert np.abs(o - O).max() <= 1e-2 and rel_l2(o, O) <= 1e-2
    np.testing.assert_allclose(host(st.lse), L, atol=2e-3)
    st2 = GpuStep(cfg, x)
    st2.score_select()
    st2.update(2, mass=dev(sel["mass"]))
    torch.cuda.synchronize()
    before = dict(k_p=x["k_p"], v_p=x["v_p"], persist_len=x["persist_len"], persist_src=x["persist_src"],
                  persist_kbar=kbar_p)
    ref = oracle.persist_update(before, sel["mass"], x["k_l"], x["v_l"], sel["kbar_l"], 0, 2, g)
    a2 = st2.state()
    for k in ("k_p", "v_p", "persist_len", "persist_src"):
        np.testing.assert_array_equal(a2[k], ref[k], err_msg=k)


def test_c344_bwd_all_heads(c344):
    cfg, x, g, kbar_p, sel = c344
    dout = synth.make_dout(cfg, seed=7)
    st = GpuStep(cfg, x)
    idx = dev(sel["topk_idx"])
    st.fwd(idx)
    gr = st.bwd(dev(dout, torch.bfloat16), idx)
    torch.cuda.synchronize()
    ref = oracle.attend_bwd(x["q"], x["k_p"], x["v_p"], x["persist_len"], x["k_l"], x["v_l"], sel["topk_idx"],
                            dout, g)
    for k in ("dq", "dk_p", "dv_p", "dk_l", "dv_l"):
        a = host(gr[k])
        err = np.abs(a - ref[k]).max()
        r = rel_l2(a, ref[k])
        print(f"[3,4,4] bwd, all heads: {k} max-abs {err:.3g} rel-L2 {r:.3g}")
        assert err <= 1e-2 and r <= 2e-2, k
