"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: the
constructor constants of the project page's usage example, closed forms,
an independent brute-force writing, torch's dense attention and autograd,
invariants of softmax attention, finite differences, and special cases of
the update rule.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def tiny_cfg(**kw):
    """Small ragged shape: 12x10 grid -> blocks of 64, 16, 32, 8 tokens."""
    c = dict(batch=1, heads=2, head_dim=8, frame_h=12, frame_w=10,
             block_t=1, block_h=8, block_w=8, chunk_frames=1,
             total_cache_size=2 * 120 + 3 * 120, local_cache_size=3 * 120,
             persistent_cache_size=2 * 120, use_local_block_sparse_attn=1,
             topk_ratio=0.25, softmax_scale=0.0, dtype="fp32",
             seed=5, plant_frac=0.2, alpha=3.0)
    c.update(kw)
    return c


def run_oracle(cfg, x, ring_head=0, step_id=0):
    g = oracle.geometry(cfg)
    kbar_p = oracle.pool_slots(x["k_p"], x["persist_len"])
    sel = oracle.score_select(x["q"], x["k_l"], ring_head, kbar_p, x["persist_len"], g)
    O, L = oracle.attend(x["q"], x["k_p"], x["v_p"], x["persist_len"], x["k_l"], x["v_l"],
                         sel["topk_idx"], g)
    state = dict(k_p=x["k_p"], v_p=x["v_p"], persist_len=x["persist_len"],
                 persist_src=x["persist_src"], persist_kbar=kbar_p)
    up = oracle.persist_update(state, sel["mass"], x["k_l"], x["v_l"], sel["kbar_l"],
                               ring_head, step_id, g)
    return g, sel, O, L, up


# ---------------------------------------------------------------------------
# B1-B3: closed forms from the project page's constructor constants
# ---------------------------------------------------------------------------


def test_geometry_closed_forms():
    gold = json.load(open(os.path.join(GOLD, "geometry_pages.json")))
    ctor, hd = gold["constructor"], gold["hand_derived"]
    g = oracle.geometry(synth.workload("decode_c1"))
    assert g.frame_tokens == hd["frame_tokens"]
    assert g.n_qblk // g.chunk_frames == hd["blocks_per_frame"]
    hist = {}
    for n in g.block_len[: hd["blocks_per_frame"]]:
        hist[str(int(n))] = hist.get(str(int(n)), 0) + 1
    assert hist == hd["block_size_histogram"]
    assert int(g.block_len[:28].sum()) == hd["frame_tokens"]
    assert g.n_qblk == hd["query_blocks"] and g.R == hd["ring_chunks"]
    assert g.n_lblk == hd["local_blocks"] and g.topk == hd["topk"]
    assert g.S == hd["persistent_slots"]
    assert ctor["max_seq_len"] == hd["max_seq_frames"] * hd["frame_tokens"]
    red = 1 - ctor["total_cache_size"] / ctor["max_seq_len"]
    assert red == pytest.approx(hd["footprint_reduction"])
    assert math.floor(100 * red) == gold["abstract_footprint_reduction_percent"]
    # every token of a frame belongs to exactly one block
    toks = np.concatenate(g.block_tok[:28])
    assert sorted(toks.tolist()) == list(range(1560))


def test_geometry_block_344():
    # [3,4,4] blocks (the project page's faster configuration) on the 30x52
    # grid: 8 block rows (7 of 4 rows + 1 of 2) x 13 block columns per
    # 3-frame group = 104 blocks of 48 (91) and 24 (13) tokens.
    g = oracle.geometry(synth.workload("decode_c1", block_t=3, block_h=4, block_w=4))
    assert (g.n_qblk, g.n_lblk, g.S, g.cap, g.topk) == (104, 208, 208, 48, 26)
    hist = {}
    for n in g.block_len:
        hist[int(n)] = hist.get(int(n), 0) + 1
    assert hist == {48: 91, 24: 13}
    assert int(g.block_len.sum()) == g.chunk_tokens == 4680
    toks = np.concatenate(g.block_tok)
    assert sorted(toks.tolist()) == list(range(4680))
    # a block spans the three frames of the chunk at the same 4x4 window
    t0 = g.block_tok[0]
    assert sorted(set((t0 // 1560).tolist())) == [0, 1, 2]


def test_geometry_tiny_config():
    g = oracle.geometry(synth.workload("tiny_fp32"))
    assert (g.n_qblk, g.R, g.n_lblk, g.S, g.topk, g.cap) == (4, 4, 16, 8, 4, 64)
    assert g.scale == pytest.approx(1 / 8)


def test_geometry_rejects_bad_sizes():
    with pytest.raises(ValueError):
        oracle.geometry(tiny_cfg(total_cache_size=1))
    with pytest.raises(ValueError):
        oracle.geometry(tiny_cfg(local_cache_size=100, total_cache_size=340))


def test_topk_rounding():
    # k = ceil(ratio * n): exact products stay put, others round up
    assert oracle.geometry(tiny_cfg(topk_ratio=0.25)).topk == 3
    assert oracle.geometry(tiny_cfg(topk_ratio=0.2)).topk == 3      # 2.4 -> 3
    assert oracle.geometry(tiny_cfg(topk_ratio=1.0)).topk == 12
    assert oracle.geometry(tiny_cfg(topk_ratio=1e-9)).topk == 1
    assert oracle.geometry(tiny_cfg(use_local_block_sparse_attn=0)).topk == 12


# ---------------------------------------------------------------------------
# F2: brute force on a tiny ragged shape
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("ring_head,sink", [(0, 0), (2, 0), (1, 2), (2, 4)])
def test_brute_force_matches(ring_head, sink):
    cfg = tiny_cfg(sink_slots=sink)
    x = synth.make_step_inputs(cfg)
    if sink:
        x["persist_len"][..., 1] = 0        # an empty sink slot is filled from the evicted chunk
        x["k_p"][..., 1, :, :] = 0
        x["v_p"][..., 1, :, :] = 0
    g, sel, O, L, up = run_oracle(cfg, x, ring_head=ring_head, step_id=7)
    br = brute.step(cfg, x["q"], x["k_l"], x["v_l"], x["k_p"], x["v_p"], x["persist_len"],
                    ring_head, 7)
    for h in range(cfg["heads"]):
        assert [list(r) for r in sel["topk_idx"][0, h]] == br["topk"][h]
        np.testing.assert_allclose(O[0, h], np.array(br["O"][h]), rtol=0, atol=1e-12)
        np.testing.assert_allclose(L[0, h], np.array(br["LSE"][h]), rtol=0, atol=1e-12)
        np.testing.assert_allclose(sel["mass"][0, h], np.array(br["mass"][h]), rtol=1e-5, atol=1e-6)
        assert int(up["n_replaced"][0, h]) == br["n_replaced"][h]
        for s, (n, src, kr, vr) in enumerate(br["slots"][h]):
            assert int(up["persist_len"][0, h, s]) == n
            if src == "empty":
                assert up["persist_src"][0, h, s] == oracle.EMPTY_SRC
            elif src is not None:
                assert int(up["persist_src"][0, h, s]) == src
            np.testing.assert_array_equal(up["k_p"][0, h, s], np.array(kr, dtype=np.float32))
            np.testing.assert_array_equal(up["v_p"][0, h, s], np.array(vr, dtype=np.float32))


# ---------------------------------------------------------------------------
# F1: ratio 1 reduces to dense softmax attention (torch fp64 SDPA / autograd)
# ---------------------------------------------------------------------------


def _dense_union(x, g, b, h):
    ks, vs = [], []
    for s in range(g.S):
        n = int(x["persist_len"][b, h, s])
        ks.append(x["k_p"][b, h, s, :n])
        vs.append(x["v_p"][b, h, s, :n])
    ks.append(x["k_l"][b, h])
    vs.append(x["v_l"][b, h])
    return np.concatenate(ks), np.concatenate(vs)


def test_ratio_one_equals_dense_attention():
    cfg = synth.workload("tiny_fp32", topk_ratio=1.0, heads=1)
    x = synth.make_step_inputs(cfg)
    g, sel, O, L, _ = run_oracle(cfg, x)
    assert sel["topk_idx"].shape[-1] == g.n_lblk
    K, V = _dense_union(x, g, 0, 0)
    qt = torch.tensor(x["q"][0, 0], dtype=torch.float64)[None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt, torch.tensor(K, dtype=torch.float64)[None, None], torch.tensor(V, dtype=torch.float64)[None, None],
        scale=g.scale)[0, 0].numpy()
    np.testing.assert_allclose(O[0, 0], ref, rtol=0, atol=1e-12)
    lse = torch.logsumexp(g.scale * qt[0, 0] @ torch.tensor(K, dtype=torch.float64).T, dim=1).numpy()
    np.testing.assert_allclose(L[0, 0], lse, rtol=0, atol=1e-12)


def test_ratio_one_backward_equals_autograd():
    cfg = tiny_cfg(topk_ratio=1.0, heads=1, plant_frac=0.0)
    x = synth.make_step_inputs(cfg)
    g = oracle.geometry(cfg)
    kbar_p = oracle.pool_slots(x["k_p"], x["persist_len"])
    sel = oracle.score_select(x["q"], x["k_l"], 0, kbar_p, x["persist_len"], g)
    dout = synth.make_dout(cfg, seed=11)
    gr = oracle.attend_bwd(x["q"], x["k_p"], x["v_p"], x["persist_len"], x["k_l"], x["v_l"],
                           sel["topk_idx"], dout, g)
    q = torch.tensor(x["q"][0, 0], dtype=torch.float64, requires_grad=True)
    kp = torch.tensor(x["k_p"][0, 0], dtype=torch.float64, requires_grad=True)
    vp = torch.tensor(x["v_p"][0, 0], dtype=torch.float64, requires_grad=True)
    kl = torch.tensor(x["k_l"][0, 0], dtype=torch.float64, requires_grad=True)
    vl = torch.tensor(x["v_l"][0, 0], dtype=torch.float64, requires_grad=True)
    lens = x["persist_len"][0, 0]
    K = torch.cat([kp[s, : int(lens[s])] for s in range(g.S)] + [kl])
    V = torch.cat([vp[s, : int(lens[s])] for s in range(g.S)] + [vl])
    o = torch.nn.functional.scaled_dot_product_attention(q[None, None], K[None, None], V[None, None],
                                                         scale=g.scale)[0, 0]
    (o * torch.tensor(dout[0, 0], dtype=torch.float64)).sum().backward()
    np.testing.assert_allclose(gr["dq"][0, 0], q.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(gr["dk_p"][0, 0], kp.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(gr["dv_p"][0, 0], vp.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(gr["dk_l"][0, 0], kl.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(gr["dv_l"][0, 0], vl.grad.numpy(), atol=1e-12)


# ---------------------------------------------------------------------------
# F3: softmax rows sum to one (LSE consistent with the attended key set)
# ---------------------------------------------------------------------------


def test_softmax_rows_sum_to_one():
    cfg = tiny_cfg(plant_frac=0.0, heads=1, head_dim=16)
    x = synth.make_step_inputs(cfg)
    g, sel, O, L, _ = run_oracle(cfg, x)
    for i in range(g.n_qblk):
        ks = [x["k_p"][0, 0, s, : x["persist_len"][0, 0, s]] for s in range(g.S)]
        ks += [x["k_l"][0, 0, g.local_tokens_of(int(p))] for p in sel["topk_idx"][0, 0, i]]
        K = np.concatenate(ks).astype(np.float64)
        for t in g.block_tok[i]:
            z = np.exp(g.scale * (K @ x["q"][0, 0, t].astype(np.float64)) - L[0, 0, t]).sum()
            assert abs(z - 1) < 1e-12


# ---------------------------------------------------------------------------
# F4: unselected blocks do not matter
# ---------------------------------------------------------------------------


def test_unselected_blocks_are_invisible():
    cfg = synth.workload("tiny_fp32")
    x = synth.make_step_inputs(cfg)
    g, sel, O, L, _ = run_oracle(cfg, x)
    rng = np.random.default_rng(0)
    for i in range(g.n_qblk):
        chosen = set(int(p) for p in sel["topk_idx"][0, 0, i])
        y = {k: v.copy() for k, v in x.items()}
        for p in range(g.n_lblk):
            if p not in chosen:
                tok = g.local_tokens_of(p)
                y["k_l"][0, 0, tok] = rng.standard_normal((len(tok), g.D)) * 50
                y["v_l"][0, 0, tok] = rng.standard_normal((len(tok), g.D)) * 50
        O2, L2 = oracle.attend(y["q"], y["k_p"], y["v_p"], y["persist_len"], y["k_l"], y["v_l"],
                               sel["topk_idx"], g, qblocks=[i])
        tok = g.block_tok[i]
        np.testing.assert_array_equal(O2[0, 0, tok], O[0, 0, tok])
        np.testing.assert_array_equal(L2[0, 0, tok], L[0, 0, tok])


def test_permuting_inside_unselected_blocks_keeps_pipeline_output():
    cfg = synth.workload("tiny_fp32")
    x = synth.make_step_inputs(cfg)
    g, sel, O, L, _ = run_oracle(cfg, x)
    rng = np.random.default_rng(1)
    union = set(int(p) for p in sel["topk_idx"].reshape(-1))
    y = {k: v.copy() for k, v in x.items()}
    for p in range(g.n_lblk):
        if p not in union:
            tok = g.local_tokens_of(p)
            perm = rng.permutation(len(tok))
            y["k_l"][:, :, tok] = x["k_l"][:, :, tok[perm]]
            y["v_l"][:, :, tok] = x["v_l"][:, :, tok[perm]]
    g2, sel2, O2, L2, _ = run_oracle(cfg, y)
    np.testing.assert_array_equal(sel2["topk_idx"], sel["topk_idx"])
    np.testing.assert_allclose(O2, O, atol=1e-12)


# ---------------------------------------------------------------------------
# F5: shift identities
# ---------------------------------------------------------------------------


def test_value_shift_and_gradient_sums():
    cfg = tiny_cfg(head_dim=16)
    x = synth.make_step_inputs(cfg)
    g, sel, O, L, _ = run_oracle(cfg, x)
    c = np.linspace(-1, 1, g.D).astype(np.float32)
    y = dict(x)
    y["v_l"] = x["v_l"] + c
    y["v_p"] = x["v_p"] + c * (np.arange(g.cap)[None, None, None, :, None] <
                               x["persist_len"][..., None, None])
    O2, _ = oracle.attend(y["q"], y["k_p"], y["v_p"], y["persist_len"], y["k_l"], y["v_l"],
                          sel["topk_idx"], g)
    np.testing.assert_allclose(O2, O + c, atol=1e-6)
    dout = synth.make_dout(cfg, seed=2)
    gr = oracle.attend_bwd(x["q"], x["k_p"], x["v_p"], x["persist_len"], x["k_l"], x["v_l"],
                           sel["topk_idx"], dout, g)
    for h in range(g.H):
        # sum over every attended key row of dK is 0; of dV is sum of dO
        sk = gr["dk_p"][0, h].sum(axis=(0, 1)) + gr["dk_l"][0, h].sum(axis=0)
        sv = gr["dv_p"][0, h].sum(axis=(0, 1)) + gr["dv_l"][0, h].sum(axis=0)
        np.testing.assert_allclose(sk, 0, atol=1e-10)
        np.testing.assert_allclose(sv, dout[0, h].astype(np.float64).sum(axis=0), atol=1e-10)
        # padding rows and unselected blocks get no gradient
        for s in range(g.S):
            n = x["persist_len"][0, h, s]
            assert not gr["dk_p"][0, h, s, n:].any() and not gr["dv_p"][0, h, s, n:].any()
        used = set(int(p) for p in sel["topk_idx"][0, h].reshape(-1))
        for p in range(g.n_lblk):
            if p not in used:
                assert not gr["dk_l"][0, h, g.local_tokens_of(p)].any()


# ---------------------------------------------------------------------------
# F6: finite differences of the backward (fp64)
# ---------------------------------------------------------------------------


def test_backward_finite_differences():
    cfg = tiny_cfg(heads=1, plant_frac=0.0)
    x = {k: (v.astype(np.float64) if v.dtype == np.float32 else v)
         for k, v in synth.make_step_inputs(cfg).items()}
    g = oracle.geometry(cfg)
    sel = oracle.score_select(x["q"], x["k_l"], 0, oracle.pool_slots(x["k_p"], x["persist_len"]),
                              x["persist_len"], g)
    idx = sel["topk_idx"]
    dout = synth.make_dout(cfg, seed=9).astype(np.float64)
    gr = oracle.attend_bwd(x["q"], x["k_p"], x["v_p"], x["persist_len"], x["k_l"], x["v_l"],
                           idx, dout, g)

    def loss(y):
        O, _ = oracle.attend(y["q"], y["k_p"], y["v_p"], y["persist_len"], y["k_l"], y["v_l"], idx, g)
        return float((O * dout).sum())

    rng = np.random.default_rng(3)
    used_local = np.concatenate([g.local_tokens_of(int(p)) for p in np.unique(idx[0, 0])])
    picks = []
    for name, grad in (("q", "dq"), ("k_l", "dk_l"), ("v_l", "dv_l")):
        for _ in range(4):
            t = int(rng.integers(x[name].shape[2])) if name == "q" else int(rng.choice(used_local))
            picks.append((name, grad, (0, 0, t, int(rng.integers(g.D)))))
    for name, grad in (("k_p", "dk_p"), ("v_p", "dv_p")):
        for _ in range(4):
            s = int(rng.integers(g.S))
            r = int(rng.integers(x["persist_len"][0, 0, s]))
            picks.append((name, grad, (0, 0, s, r, int(rng.integers(g.D)))))
    eps = 1e-5
    for name, grad, ix in picks:
        y = dict(x)
        y[name] = x[name].copy()
        y[name][ix] += eps
        lp = loss(y)
        y[name][ix] -= 2 * eps
        lm = loss(y)
        fd = (lp - lm) / (2 * eps)
        an = gr[grad][ix]
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, ix, fd, an)


# ---------------------------------------------------------------------------
# Masses: each query block's softmax sums to one
# ---------------------------------------------------------------------------


def test_masses_sum_to_query_block_count():
    cfg = synth.workload("tiny_fp32")
    x = synth.make_step_inputs(cfg)
    g, sel, *_ = run_oracle(cfg, x)
    np.testing.assert_allclose(sel["mass"].sum(axis=-1), g.n_qblk, rtol=1e-5)
    # identical pooled keys everywhere -> uniform masses
    qbar = sel["qbar"]
    kb = np.ones((g.B, g.H, g.n_lblk, g.D), np.float32)
    kp = np.ones((g.B, g.H, g.S, g.D), np.float32)
    m = oracle.pooled_mass(qbar, kp, x["persist_len"], kb, g)
    np.testing.assert_allclose(m, g.n_qblk / (g.S + g.n_lblk), rtol=1e-5)


# ---------------------------------------------------------------------------
# Selection tie rule and planted separation (F8)
# ---------------------------------------------------------------------------


def test_exact_ties_go_to_lower_logical_index():
    cfg = tiny_cfg(plant_frac=0.0, heads=1)
    g = oracle.geometry(cfg)
    scores = np.zeros((1, 1, g.n_qblk, g.n_lblk), np.float32)   # every block ties
    for rh in range(g.R):
        idx = oracle.select_topk(scores, g, rh)
        # the oldest chunk is physical slot rh; its first k blocks win
        expect = sorted(rh * g.n_qblk + e for e in range(g.topk))
        assert all(list(r) == expect for r in idx[0, 0])


def test_planted_blocks_are_selected():
    cfg = synth.workload("tiny_fp32", plant_frac=0.0, heads=1)
    g = oracle.geometry(cfg)
    x = synth.make_step_inputs(cfg)
    rng = np.random.default_rng(4)
    u = rng.standard_normal(g.D)
    u /= np.linalg.norm(u)
    planted = sorted(rng.choice(g.n_lblk, size=g.topk, replace=False).tolist())
    for p in planted:
        x["k_l"][0, 0, g.local_tokens_of(p)] += 40 * u
    x["q"][0, 0] += 5 * u
    sel = oracle.score_select(x["q"], x["k_l"], 1, oracle.pool_slots(x["k_p"], x["persist_len"]),
                              x["persist_len"], g)
    assert all(list(r) == planted for r in sel["topk_idx"][0, 0])


# ---------------------------------------------------------------------------
# F7: update special cases
# ---------------------------------------------------------------------------


def _state(x, g):
    return dict(k_p=x["k_p"], v_p=x["v_p"], persist_len=x["persist_len"],
                persist_src=x["persist_src"], persist_kbar=oracle.pool_slots(x["k_p"], x["persist_len"]))


def test_update_keeps_state_when_entrants_lose():
    cfg = synth.workload("tiny_fp32")
    x = synth.make_step_inputs(cfg)
    g = oracle.geometry(cfg)
    mass = np.zeros((g.B, g.H, g.S + g.n_lblk), np.float32)
    mass[..., : g.S] = 1.0
    st = _state(x, g)
    kbl = oracle.pool_local_blocks(x["k_l"], g)
    up = oracle.persist_update(st, mass, x["k_l"], x["v_l"], kbl, 0, 3, g)
    for k in ("k_p", "v_p", "persist_len", "persist_src", "persist_kbar"):
        np.testing.assert_array_equal(up[k], st[k])
    assert not up["n_replaced"].any() and up["ring_head"] == 1


def test_update_fills_empty_cache_in_order():
    cfg = synth.workload("tiny_fp32")
    x = synth.make_step_inputs(cfg)
    g = oracle.geometry(cfg)
    st = _state(x, g)
    st["persist_len"] = np.zeros_like(st["persist_len"])
    st["k_p"] = np.zeros_like(st["k_p"])
    st["v_p"] = np.zeros_like(st["v_p"])
    mass = np.random.default_rng(0).random((g.B, g.H, g.S + g.n_lblk)).astype(np.float32)
    kbl = oracle.pool_local_blocks(x["k_l"], g)
    rh = 2
    up = oracle.persist_update(st, mass, x["k_l"], x["v_l"], kbl, rh, 5, g)
    ne = g.n_qblk                        # every evicted block fits
    assert (up["n_replaced"] == ne).all()
    for b in range(g.B):
        for h in range(g.H):
            for e in range(ne):
                tok = rh * g.chunk_tokens + g.block_tok[e]
                np.testing.assert_array_equal(up["k_p"][b, h, e, : len(tok)], x["k_l"][b, h, tok])
                assert up["persist_src"][b, h, e] == 5 * g.n_qblk + e
            assert (up["persist_len"][b, h, ne:] == 0).all()
            assert (up["persist_src"][b, h, ne:] == oracle.EMPTY_SRC).all()


def test_update_replaces_exactly_the_planted_count():
    cfg = synth.workload("tiny_fp32")
    x = synth.make_step_inputs(cfg)
    g = oracle.geometry(cfg)
    rng = np.random.default_rng(8)
    for r in range(0, g.n_qblk + 1):
        mass = rng.uniform(1.0, 2.0, (g.B, g.H, g.S + g.n_lblk)).astype(np.float32)
        old = 1
        ev = slice(g.S + old * g.n_qblk, g.S + (old + 1) * g.n_qblk)
        mass[..., ev] = 0.5
        winners = rng.choice(g.n_qblk, size=r, replace=False)
        losers = rng.choice(g.S, size=r, replace=False)
        mass[..., g.S + old * g.n_qblk + winners] = 5.0
        mass[..., losers] = 0.1
        up = oracle.persist_update(_state(x, g), mass, x["k_l"], x["v_l"],
                                   oracle.pool_local_blocks(x["k_l"], g), old, 1, g)
        assert (up["n_replaced"] == r).all()
        assert sorted(np.nonzero(~up["keep"][0, 0])[0].tolist()) == sorted(losers.tolist())


def test_update_valid_count_and_src_multiset():
    cfg = synth.workload("tiny_fp32")
    x = synth.make_step_inputs(cfg)
    g = oracle.geometry(cfg)
    rng = np.random.default_rng(9)
    st = _state(x, g)
    st["persist_len"] = st["persist_len"].copy()
    st["persist_len"][..., ::3] = 0                 # some empty slots
    nvalid = (st["persist_len"] > 0).sum(-1)
    mass = rng.random((g.B, g.H, g.S + g.n_lblk)).astype(np.float32)
    rh = 3
    up = oracle.persist_update(st, mass, x["k_l"], x["v_l"], oracle.pool_local_blocks(x["k_l"], g),
                               rh, 2, g)
    after = (up["persist_len"] > 0).sum(-1)
    np.testing.assert_array_equal(after, np.minimum(g.S, nvalid + g.n_qblk))
    for b in range(g.B):
        for h in range(g.H):
            cands = [(-float(mass[b, h, s]), 0, s) for s in range(g.S) if st["persist_len"][b, h, s]]
            cands += [(-float(mass[b, h, g.S + rh * g.n_qblk + e]), 1, e) for e in range(g.n_qblk)]
            top = sorted(cands)[: g.S]
            expect = sorted([int(st["persist_src"][b, h, c[2]]) if c[1] == 0 else 2 * g.n_qblk + c[2]
                             for c in top])
            got = sorted(int(v) for v in up["persist_src"][b, h] if v != oracle.EMPTY_SRC)
            assert got == expect


def test_sink_slots_stay_under_lowest_mass():
    cfg = dict(synth.workload("tiny_fp32"), sink_slots=2)
    x = synth.make_step_inputs(cfg)
    g = oracle.geometry(cfg)
    assert g.n_sink == 2
    rng = np.random.default_rng(12)
    mass = rng.uniform(1.0, 2.0, (g.B, g.H, g.S + g.n_lblk)).astype(np.float32)
    n = min(g.n_qblk, g.S - 2)
    mass[..., :2] = 0.0                       # sinks receive nothing
    mass[..., 2:2 + n] = 0.01                 # the n weakest other incumbents
    old = 0
    mass[..., g.S + old * g.n_qblk:g.S + (old + 1) * g.n_qblk] = 50.0
    st = _state(x, g)
    up = oracle.persist_update(st, mass, x["k_l"], x["v_l"], oracle.pool_local_blocks(x["k_l"], g), old, 1, g)
    for k in ("k_p", "v_p", "persist_len", "persist_src", "persist_kbar"):
        np.testing.assert_array_equal(up[k][:, :, :2], st[k][:, :, :2])
    # the evicted blocks all win, against the weakest non-sink incumbents
    assert (up["n_replaced"] == n).all()
    assert (~up["keep"][..., 2:2 + n]).all() and up["keep"][..., 2 + n:].all()
    # without sinks the two zero-mass slots are the first to go
    up0 = oracle.persist_update(st, mass, x["k_l"], x["v_l"], oracle.pool_local_blocks(x["k_l"], g), old, 1,
                                oracle.geometry(dict(cfg, sink_slots=0)))
    assert (~up0["keep"][..., :2]).all()


def test_sink_fill_from_empty_cache():
    cfg = dict(synth.workload("tiny_fp32"), sink_slots=3)
    x = synth.make_step_inputs(cfg)
    g = oracle.geometry(cfg)
    st = _state(x, g)
    for k in ("persist_len", "k_p", "v_p", "persist_kbar"):
        st[k] = np.zeros_like(st[k])
    st["persist_src"] = np.full_like(st["persist_src"], oracle.EMPTY_SRC)
    mass = np.zeros((g.B, g.H, g.S + g.n_lblk), np.float32)
    rh = 1
    mass[..., g.S + rh * g.n_qblk + 0] = 9.0   # block 0 would win anyway; blocks 1, 2 have no mass
    kbl = oracle.pool_local_blocks(x["k_l"], g)
    up = oracle.persist_update(st, mass, x["k_l"], x["v_l"], kbl, rh, 4, g)
    for b in range(g.B):
        for h in range(g.H):
            for s in range(3):                     # sink slot s holds evicted block s
                tok = rh * g.chunk_tokens + g.block_tok[s]
                np.testing.assert_array_equal(up["k_p"][b, h, s, :len(tok)], x["k_l"][b, h, tok])
                assert up["persist_src"][b, h, s] == 4 * g.n_qblk + s
                np.testing.assert_array_equal(up["persist_kbar"][b, h, s], kbl[b, h, rh * g.n_qblk + s])
            # the remaining blocks fill slots 3.. in ascending order
            rest = list(range(3, g.n_qblk))
            for j, e in enumerate(rest):
                assert up["persist_src"][b, h, 3 + j] == 4 * g.n_qblk + e
    assert (up["n_replaced"] == g.n_qblk).all()


def test_near_tie_band():
    s = np.array([3.0, 2.0, 1.00000001, 1.0, 0.0])
    nt, band, _ = oracle.near_tie_rows(s, 3)
    assert nt and band == pytest.approx(3e-4)
    nt, _, _ = oracle.near_tie_rows(s, 2)
    assert not nt


# ---------------------------------------------------------------------------
# Token-exact masses (reading R19)
# ---------------------------------------------------------------------------


def _sel_for(cfg, x, ring_head=0):
    g = oracle.geometry(cfg)
    sel = oracle.score_select(x["q"], x["k_l"], ring_head, oracle.pool_slots(x["k_p"], x["persist_len"]),
                              x["persist_len"], g)
    return g, sel


@pytest.mark.parametrize("ring_head", [0, 1])
def test_token_mass_totals_and_zeros(ring_head):
    cfg = tiny_cfg()
    x = synth.make_step_inputs(cfg)
    x["persist_len"][0, 1, 0] = 0          # one empty slot
    g, sel = _sel_for(cfg, x, ring_head)
    m = oracle.token_mass(x["q"], x["k_p"], x["persist_len"], x["k_l"], sel["topk_idx"], g)
    # every query token's probabilities sum to one
    np.testing.assert_allclose(m.sum(axis=-1, dtype=np.float64), g.chunk_tokens, rtol=1e-6)
    assert m[0, 1, 0] == 0
    for b in range(g.B):
        for h in range(g.H):
            chosen = set(np.unique(sel["topk_idx"][b, h]).tolist())
            for p in range(g.n_lblk):
                assert (m[b, h, g.S + p] > 0) == (p in chosen), (b, h, p)


def test_token_mass_equals_value_gradient_of_unit_upstream():
    """With dO = 1 the value gradient of a key row is the probability mass it
    receives (dV = P^T dO), so per-block sums of the (finite-difference
    pinned) backward equal the token-exact masses."""
    cfg = tiny_cfg(heads=2)
    x = synth.make_step_inputs(cfg)
    g, sel = _sel_for(cfg, x)
    idx = sel["topk_idx"]
    ones = np.ones((g.B, g.H, g.chunk_tokens, g.D))
    gr = oracle.attend_bwd(x["q"], x["k_p"], x["v_p"], x["persist_len"], x["k_l"], x["v_l"], idx, ones, g)
    m = oracle.token_mass(x["q"], x["k_p"], x["persist_len"], x["k_l"], idx, g)
    ref = np.zeros_like(m, dtype=np.float64)
    ref[..., :g.S] = gr["dv_p"][..., 3].sum(axis=-1)
    for p in range(g.n_lblk):
        ref[..., g.S + p] = gr["dv_l"][:, :, g.local_tokens_of(p), 3].sum(axis=-1)
    np.testing.assert_allclose(m, ref, rtol=1e-6, atol=1e-9)


def test_token_mass_uniform_keys_closed_form():
    """All key rows identical -> each query spreads its mass uniformly over its
    N_t keys: slot s gets sum_t len_s / N_t, local block p gets
    sum over query tokens whose block selected p of len_p / N_t."""
    cfg = tiny_cfg(plant_frac=0.0)
    x = synth.make_step_inputs(cfg)
    g, sel = _sel_for(cfg, x)
    idx = sel["topk_idx"]
    kp = np.ones_like(x["k_p"]) * 0.5
    kl = np.ones_like(x["k_l"]) * 0.5
    m = oracle.token_mass(x["q"], kp, x["persist_len"], kl, idx, g)
    blen = g.block_len
    for b in range(g.B):
        for h in range(g.H):
            plen = x["persist_len"][b, h].astype(np.float64)
            exp = np.zeros(g.S + g.n_lblk)
            for i in range(g.n_qblk):
                n_t = plen.sum() + sum(blen[p % g.n_qblk] for p in idx[b, h, i])
                nq = blen[i]
                exp[:g.S] += nq * plen / n_t
                for p in idx[b, h, i]:
                    exp[g.S + p] += nq * blen[p % g.n_qblk] / n_t
            np.testing.assert_allclose(m[b, h], exp, rtol=1e-6)


# ---------------------------------------------------------------------------
# The local ring and the per-chunk schedule (training-algorithm fragment:
# denoising passes attend the current chunk; the cache pass attends and
# updates)
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("ring_head", [0, 1, 2, 3])
def test_ring_append_writes_the_newest_logical_chunk(ring_head):
    """The appended chunk becomes the newest logical chunk, whatever the ring
    phase: block e of it is logical block (R-1)*n_qblk + e, whose tokens hold
    the new rows; every other token keeps its value."""
    cfg = synth.workload("tiny_fp32")
    g = oracle.geometry(cfg)
    x = synth.make_step_inputs(cfg)
    rng = np.random.default_rng(ring_head)
    kn = rng.standard_normal(x["q"].shape).astype(np.float32)
    vn = rng.standard_normal(x["q"].shape).astype(np.float32)
    k2, v2 = oracle.ring_append(x["k_l"], x["v_l"], kn, vn, ring_head, g)
    touched = np.zeros(x["k_l"].shape[2], bool)
    for p in range(g.n_lblk):
        lg = g.logical_of(p, ring_head)
        if lg >= (g.R - 1) * g.n_qblk:
            e = lg - (g.R - 1) * g.n_qblk
            tok = g.local_tokens_of(p)
            np.testing.assert_array_equal(k2[:, :, tok], kn[:, :, g.block_tok[e]])
            np.testing.assert_array_equal(v2[:, :, tok], vn[:, :, g.block_tok[e]])
            touched[tok] = True
    assert touched.sum() == g.chunk_tokens
    np.testing.assert_array_equal(k2[:, :, ~touched], x["k_l"][:, :, ~touched])
    np.testing.assert_array_equal(v2[:, :, ~touched], x["v_l"][:, :, ~touched])


def _schedule_inputs(cfg, n_passes, seed):
    rng = np.random.default_rng(seed)
    shape = synth.make_step_inputs(cfg)["q"].shape
    return [tuple(rng.standard_normal(shape).astype(np.float32) for _ in range(3)) for _ in range(n_passes)]


def test_every_pass_attends_its_own_chunk():
    """A block planted (large alpha along u, queries leaning on u) in the keys
    of one pass is selected by every query block of that pass and by no
    other pass: each pass scores the local window that holds its own keys,
    not those of the pass before it or the chunk the last update evicted."""
    cfg = synth.workload("tiny_fp32", plant_frac=0.0, heads=1)
    g = oracle.geometry(cfg)
    x = synth.make_step_inputs(cfg)
    rng = np.random.default_rng(11)
    u = rng.standard_normal(g.D)
    u /= np.linalg.norm(u)
    passes = _schedule_inputs(cfg, 3, 12)
    ring_head = 2
    newest = (ring_head + g.R - 1) % g.R
    # pass i plants block i of its chunk and pushes the blocks the other
    # passes plant far down (-alpha u), so a stale window would show
    assert len(passes) <= g.n_qblk
    planted = [newest * g.n_qblk + i for i in range(len(passes))]
    for i, (q, k, v) in enumerate(passes):
        for j in range(len(passes)):
            k[0, 0, g.block_tok[j]] += (60 if j == i else -60) * u
        q[0, 0] += 6 * u
    out = oracle.decode_chunk(_state(x, g), x["k_l"], x["v_l"], passes, ring_head, 4, g)
    for i, r in enumerate(out["passes"]):
        idx = r["sel"]["topk_idx"][0, 0]
        assert all(planted[i] in row for row in idx), i
        assert all(planted[j] not in row for row in idx for j in range(len(passes)) if j != i), i


def test_denoising_passes_do_not_touch_the_update():
    """The persistent state after a chunk depends on the cache pass only: the
    same chunk with zero or three denoising passes before its cache pass
    gives the same update, and the ring ends with the cache pass's keys."""
    cfg = synth.workload("tiny_fp32", heads=2)
    g = oracle.geometry(cfg)
    x = synth.make_step_inputs(cfg)
    passes = _schedule_inputs(cfg, 4, 13)
    a = oracle.decode_chunk(_state(x, g), x["k_l"], x["v_l"], passes, 1, 7, g)
    b = oracle.decode_chunk(_state(x, g), x["k_l"], x["v_l"], passes[-1:], 1, 7, g)
    for k in ("k_p", "v_p", "persist_len", "persist_src", "persist_kbar", "n_replaced"):
        np.testing.assert_array_equal(a["update"][k], b["update"][k])
    np.testing.assert_array_equal(a["k_l"], b["k_l"])
    assert a["update"]["ring_head"] == 2
    # the evicted chunk's rows went into the persistent cache, not a denoising pass's rows
    for bb in range(g.B):
        for h in range(g.H):
            for s in range(g.S):
                src = a["update"]["persist_src"][bb, h, s]
                if src >= 7 * g.n_qblk:
                    e = src - 7 * g.n_qblk
                    tok = 1 * g.chunk_tokens + g.block_tok[e]
                    n = len(tok)
                    np.testing.assert_array_equal(a["update"]["k_p"][bb, h, s, :n], x["k_l"][bb, h, tok])
