"""GPU parity of the token-exact attention mass (pbsa_fwd_mass) and of the
persistent update driven by it, against the oracle's token_mass.

Masses: the GPU sums fp32 exponentials of fp32 scores of the same
bf16-rounded inputs the oracle takes in float64, so they agree to rounding:
|gpu - oracle| <= 1e-4 * (1 + |oracle|).  Empty slots and unselected local
blocks are exactly 0 on both sides.  The forward outputs of pbsa_fwd_mass are
those of pbsa_fwd up to rounding (the summation order over the persistent
keys differs).  Update decisions are exact except counted near
ties of the oracle's masses; the moved state is bit-exact given the decisions.
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_15_amd as pb
import oracle
import synth
from pbsa_harness import GpuStep, compare_update_decisions, decisions_from_state, dev, host, rel_l2
from test_gpu_parity import SMALL, oracle_select

pytestmark = pytest.mark.gpu


def check_mass(m_gpu, m_ora, g, topk, plen, label):
    err = np.abs(m_gpu.astype(np.float64) - m_ora) / (1.0 + np.abs(m_ora))
    print(f"{label}: token mass max scaled error {err.max():.3g}")
    assert err.max() <= 1e-4
    np.testing.assert_allclose(m_gpu.sum(-1, dtype=np.float64), g.chunk_tokens, rtol=1e-4)
    for b in range(m_gpu.shape[0]):
        for h in range(m_gpu.shape[1]):
            assert (m_gpu[b, h, :g.S][plen[b, h] == 0] == 0).all()
            unsel = np.setdiff1d(np.arange(g.n_lblk), np.unique(topk[b, h]))
            assert (m_gpu[b, h, g.S + unsel] == 0).all()


def small_inputs(name):
    cfg = SMALL[name]
    x = synth.make_step_inputs(cfg)
    if name == "ragged_bf16":
        x["persist_len"][..., ::5] = 0
        x["k_p"][..., ::5, :, :] = 0
        x["v_p"][..., ::5, :, :] = 0
    return cfg, x


@pytest.mark.parametrize("name", list(SMALL))
def test_fwd_mass_small(name):
    cfg, x = small_inputs(name)
    g, _, sel = oracle_select(cfg, x, 0)
    ref = oracle.token_mass(x["q"], x["k_p"], x["persist_len"], x["k_l"], sel["topk_idx"], g)
    st = GpuStep(cfg, x)
    idx = dev(sel["topk_idx"])
    st.fwd(idx)
    torch.cuda.synchronize()
    o1, l1 = st.o.clone(), st.lse.clone()
    st.fwd_mass(idx)
    torch.cuda.synchronize()
    # the same attention; the plain forward adds the persistent keys in packed
    # 64-key steps, this one slot by slot, so they agree to rounding
    o_a, o_b = host(o1), host(st.o)
    assert np.abs(o_a - o_b).max() <= 2e-3 and rel_l2(o_b, o_a) <= 1e-3, name
    np.testing.assert_allclose(host(st.lse), host(l1), rtol=0, atol=1e-4)
    check_mass(host(st.mass), ref, g, sel["topk_idx"], x["persist_len"], name)


@pytest.mark.parametrize("name", ["ragged_bf16", "ragged_fp32", "block344_bf16"])
@pytest.mark.parametrize("ring_head", [0, 1])
def test_token_mass_update_small(name, ring_head):
    cfg, x = small_inputs(name)
    x["ring_head"][:] = ring_head
    g, kbar_p, sel = oracle_select(cfg, x, ring_head)
    ref_m = oracle.token_mass(x["q"], x["k_p"], x["persist_len"], x["k_l"], sel["topk_idx"], g)
    before = dict(k_p=x["k_p"], v_p=x["v_p"], persist_len=x["persist_len"], persist_src=x["persist_src"],
                  persist_kbar=kbar_p)
    step_id = 2
    ref = oracle.persist_update(before, ref_m, x["k_l"], x["v_l"], sel["kbar_l"], ring_head, step_id, g)
    st = GpuStep(cfg, x)
    st.score_select()
    st.fwd_mass()
    st.update(step_id)
    torch.cuda.synchronize()
    after = st.state()
    keep_g, admit_g = decisions_from_state(before, after, step_id, g.n_qblk)
    nd = compare_update_decisions(keep_g, admit_g, ref["keep"], ref["admit"], ref_m, x["persist_len"],
                                  ring_head, g)
    print(f"{name}: token-mass update, near-tie heads {nd}, admitted {admit_g.sum(-1).tolist()}")
    moved = oracle.apply_update(dict(before, persist_kbar=host(GpuStep(cfg, x).pkbar)), keep_g, admit_g,
                                x["k_l"], x["v_l"], host(st.kbar_l), ring_head, step_id, g)
    for k in ("k_p", "v_p", "persist_len", "persist_src", "persist_kbar"):
        np.testing.assert_array_equal(after[k], moved[k], err_msg=k)


def test_c1_token_mass_and_update():
    cfg = synth.workload("decode_c1")
    x = synth.make_step_inputs(cfg)
    g, kbar_p, sel = oracle_select(cfg, x, 0)
    st = GpuStep(cfg, x)
    st.score_select()
    st.fwd_mass(dev(sel["topk_idx"]))
    torch.cuda.synchronize()
    m_gpu = host(st.mass)
    heads = list(range(g.H))      # every head
    c2 = dict(cfg, heads=len(heads))
    g2 = oracle.geometry(c2)
    xs = {k: v[:, heads] for k, v in x.items() if k != "ring_head"}
    ref_m = oracle.token_mass(xs["q"], xs["k_p"], xs["persist_len"], xs["k_l"], sel["topk_idx"][:, heads], g2)
    check_mass(m_gpu[:, heads], ref_m, g2, sel["topk_idx"][:, heads], xs["persist_len"], "decode_c1")
    # the update on those heads against the oracle's decisions from its own masses
    step_id = 4
    before = dict(k_p=x["k_p"], v_p=x["v_p"], persist_len=x["persist_len"], persist_src=x["persist_src"],
                  persist_kbar=kbar_p)
    st.update(step_id)
    torch.cuda.synchronize()
    after = st.state()
    keep_g, admit_g = decisions_from_state(before, after, step_id, g.n_qblk)
    keep_o, admit_o = oracle.update_decisions(ref_m, xs["persist_len"], 0, g2)
    nd = compare_update_decisions(keep_g[:, heads], admit_g[:, heads], keep_o, admit_o, ref_m, xs["persist_len"],
                                  0, g2)
    print(f"decode_c1 token-mass update: admitted per head {admit_g.sum(-1).tolist()}, near-tie heads {nd}")
