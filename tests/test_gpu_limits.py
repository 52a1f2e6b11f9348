"""GPU parity at the plan's size limits: 2048 query blocks per chunk, 2048
local blocks and 2048 persistent slots (a 60x60 frame grid with ragged edge
blocks, 32-frame chunks, one-chunk ring, head_dim 64, bf16).

The oracle runs the whole selection, the update decisions and the data
movement; attention and dQ are checked on sampled query blocks; dK / dV by
identities that hold at any size (over every key, sum dK = 0 and sum dV =
sum of dO); token-exact masses by their per-head total.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from pbsa_harness import GpuStep, compare_topk, compare_update_decisions, decisions_from_state, dev, host, rel_l2

pytestmark = pytest.mark.gpu

FT = 60 * 60


def max_cfg():
    return dict(batch=1, heads=1, head_dim=64, frame_h=60, frame_w=60, block_t=1, block_h=8, block_w=8,
                chunk_frames=32, total_cache_size=2 * 32 * FT, local_cache_size=32 * FT,
                persistent_cache_size=32 * FT, use_local_block_sparse_attn=1, topk_ratio=0.125,
                softmax_scale=0.0, dtype="bf16", seed=41, plant_frac=0.02, alpha=4.0)


@pytest.fixture(scope="module")
def lim():
    cfg = max_cfg()
    g = oracle.geometry(cfg)
    assert (g.n_qblk, g.n_lblk, g.S, g.topk) == (2048, 2048, 2048, 256)
    x = synth.make_step_inputs(cfg)
    kbar_p = oracle.pool_slots(x["k_p"], x["persist_len"])
    sel = oracle.score_select(x["q"], x["k_l"], 0, kbar_p, x["persist_len"], g)
    return cfg, g, x, kbar_p, sel


def test_limits_select_fwd_bwd(lim):
    cfg, g, x, kbar_p, sel = lim
    st = GpuStep(cfg, x)
    st.score_select()
    torch.cuda.synchronize()
    nb, nm = compare_topk(host(st.topk), sel["topk_idx"], sel["scores"], g.topk)
    print(f"limits: near-tie rows {nb}, mismatched rows {nm}")
    np.testing.assert_allclose(host(st.mass), sel["mass"], rtol=1e-4, atol=1e-5)
    idx = dev(sel["topk_idx"])
    st.fwd(idx)
    dout = synth.make_dout(cfg, seed=43)
    gr = st.bwd(dev(dout, torch.bfloat16), idx)
    torch.cuda.synchronize()
    blocks = [0, 7, 1000, 2047]
    O, L = oracle.attend(x["q"], x["k_p"], x["v_p"], x["persist_len"], x["k_l"], x["v_l"], sel["topk_idx"], g,
                         qblocks=blocks)
    rows = np.concatenate([g.block_tok[i] for i in blocks])
    o = host(st.o)[:, :, rows]
    assert np.abs(o - O[:, :, rows]).max() <= 1e-2 and rel_l2(o, O[:, :, rows]) <= 1e-2
    np.testing.assert_allclose(host(st.lse)[:, :, rows], L[:, :, rows], atol=2e-3)
    ref = oracle.attend_bwd(x["q"], x["k_p"], x["v_p"], x["persist_len"], x["k_l"], x["v_l"], sel["topk_idx"],
                            dout, g, qblocks=[7, 2047])
    r2 = np.concatenate([g.block_tok[i] for i in (7, 2047)])
    dq = host(gr["dq"])
    assert np.isfinite(dq).all()
    assert np.abs(dq[:, :, r2] - ref["dq"][:, :, r2]).max() <= 1e-2 and rel_l2(dq[:, :, r2], ref["dq"][:, :, r2]) <= 2e-2
    dk = np.concatenate([host(gr["dk_p"]).reshape(-1, g.D), host(gr["dk_l"]).reshape(-1, g.D)]).astype(np.float64)
    dv = np.concatenate([host(gr["dv_p"]).reshape(-1, g.D), host(gr["dv_l"]).reshape(-1, g.D)]).astype(np.float64)
    assert np.isfinite(dk).all() and np.isfinite(dv).all()
    assert np.abs(dk.sum(0)).max() <= 1e-3 * np.abs(dk).sum(0).max()
    want = dout.astype(np.float64).reshape(-1, g.D).sum(0)
    assert np.abs(dv.sum(0) - want).max() <= 1e-2 * np.abs(want).max() + 1e-2


def test_limits_update_and_token_mass(lim):
    cfg, g, x, kbar_p, sel = lim
    step_id = 1
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
    moved = oracle.apply_update(dict(before, persist_kbar=host(GpuStep(cfg, x).pkbar)), keep_g, admit_g,
                                x["k_l"], x["v_l"], host(st.kbar_l), 0, step_id, g)
    for k in ("k_p", "v_p", "persist_len", "persist_src", "persist_kbar"):
        np.testing.assert_array_equal(after[k], moved[k], err_msg=k)
    print(f"limits update: admitted {admit_g.sum()}, near-tie heads {nd}")
    st2 = GpuStep(cfg, x)
    st2.score_select()
    st2.fwd_mass()
    torch.cuda.synchronize()
    m = host(st2.mass).astype(np.float64)
    assert (m >= 0).all()
    np.testing.assert_allclose(m.sum(-1), g.chunk_tokens, rtol=1e-4)
