"""GPU parity of the sink pattern (pinned leading persistent slots) and of a
rollout that starts from an empty persistent cache, with pooled and with
token-exact masses, against the oracle (teacher-forced: every step the oracle
starts from the GPU's pre-step state)."""
import numpy as np
import pytest
import torch

import block_sparse_attention_15_amd as pb
from block_sparse_attention_15_amd.rollout import DecodeLoop
import oracle
import synth
from pbsa_harness import GpuStep, compare_topk, compare_update_decisions, decisions_from_state, dev, host
from test_gpu_parity import SMALL, oracle_select

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("ring_head", [0, 1])
@pytest.mark.parametrize("name", ["ragged_bf16", "ragged_fp32", "block344_bf16"])
def test_sink_update(name, ring_head):
    cfg = dict(SMALL[name], sink_slots=4)
    x = synth.make_step_inputs(cfg)
    x["ring_head"][:] = ring_head
    for s in (1, 6):                      # an empty sink slot and an empty ordinary slot
        x["persist_len"][..., s] = 0
        x["k_p"][..., s, :, :] = 0
        x["v_p"][..., s, :, :] = 0
    g, kbar_p, sel = oracle_select(cfg, x, ring_head)
    assert g.n_sink == 4
    step_id = 3
    before = dict(k_p=x["k_p"], v_p=x["v_p"], persist_len=x["persist_len"], persist_src=x["persist_src"],
                  persist_kbar=kbar_p)
    ref = oracle.persist_update(before, sel["mass"], x["k_l"], x["v_l"], sel["kbar_l"], ring_head, step_id, g)
    st = GpuStep(cfg, x)
    st.score_select()
    st.update(step_id)
    torch.cuda.synchronize()
    after = st.state()
    keep_g, admit_g = decisions_from_state(before, after, step_id, g.n_qblk)
    nd = compare_update_decisions(keep_g, admit_g, ref["keep"], ref["admit"], sel["mass"], x["persist_len"],
                                  ring_head, g)
    moved = oracle.apply_update(dict(before, persist_kbar=host(GpuStep(cfg, x).pkbar)), keep_g, admit_g,
                                x["k_l"], x["v_l"], host(st.kbar_l), ring_head, step_id, g)
    for k in ("k_p", "v_p", "persist_len", "persist_src", "persist_kbar"):
        np.testing.assert_array_equal(after[k], moved[k], err_msg=k)
    np.testing.assert_array_equal(host(st.n_rep), admit_g.sum(-1))
    # sink slot 1 took evicted block 1; valid sink slots are untouched
    assert (after["persist_src"][..., 1] == step_id * g.n_qblk + 1).all()
    for s in (0, 2, 3):
        np.testing.assert_array_equal(after["k_p"][..., s, :, :], x["k_p"][..., s, :, :])
    # pure data movement with the oracle's masses
    st2 = GpuStep(cfg, x)
    st2.score_select()
    st2.update(step_id, mass=dev(sel["mass"]))
    torch.cuda.synchronize()
    a2 = st2.state()
    for k in ("k_p", "v_p", "persist_len", "persist_src"):
        np.testing.assert_array_equal(a2[k], ref[k], err_msg=k)
    np.testing.assert_array_equal(host(st2.n_rep), ref["n_replaced"])
    print(f"{name}: sink update, near-tie heads {nd}")


def empty_loop(cfg, prev, mass):
    p = pb.pbsa_plan(cfg)
    cache = pb.PBSACache(p)                # zero rows, len 0 everywhere
    cache.persist_src.fill_(int(oracle.EMPTY_SRC))
    dt = p.torch_dtype
    ct = p.chunk_tokens
    cache.k_local[:, :, :ct].copy_(dev(prev["k"], dt))
    cache.v_local[:, :, :ct].copy_(dev(prev["v"], dt))
    cache.refresh_pooled_keys()
    return p, cache, DecodeLoop(p, cache, mass=mass)


@pytest.mark.parametrize("mass", ["pooled", "token"])
def test_rollout_from_empty_cache_with_sinks(mass):
    base = SMALL["ragged_bf16"]
    nq_frame = 6                           # blocks per 14x22 frame
    cfg = dict(base, sink_slots=nq_frame, steps=12, plant_blocks=2, drift_p=0.25, redraw_every=5, seed=31)
    g = oracle.geometry(cfg)
    stream = synth.RolloutStream(cfg)
    prev = stream.chunk(-1)
    p, cache, loop = empty_loop(cfg, prev, mass)
    dt = p.torch_dtype
    _, _, warm = empty_loop(cfg, prev, mass)
    ch0 = stream.chunk(0)
    warm.load_chunk(dev(ch0["q"], dt), dev(ch0["k"], dt), dev(ch0["v"], dt))
    warm.step()
    torch.cuda.synchronize()
    loop.capture()
    chunks = [prev]
    sink_src = None
    tot_heads = 0
    for s in range(cfg["steps"]):
        ch = stream.chunk(s)
        chunks = [chunks[-1], ch]
        rh = int(host(cache.ring_head)[0])
        before = dict(k_p=host(cache.k_pers), v_p=host(cache.v_pers), persist_len=host(cache.persist_len),
                      persist_src=host(cache.persist_src), persist_kbar=host(cache.persist_kbar))
        loop.load_chunk(dev(ch["q"], dt), dev(ch["k"], dt), dev(ch["v"], dt))
        loop.replay()
        torch.cuda.synchronize()
        k_l = np.zeros((g.B, g.H, g.R * g.chunk_tokens, g.D), np.float32)
        v_l = np.zeros_like(k_l)
        for logical, c in enumerate(chunks):
            slot = (rh + logical) % g.R
            k_l[:, :, slot * g.chunk_tokens:(slot + 1) * g.chunk_tokens] = c["k"]
            v_l[:, :, slot * g.chunk_tokens:(slot + 1) * g.chunk_tokens] = c["v"]
        sel = oracle.score_select(ch["q"], k_l, rh, before["persist_kbar"], before["persist_len"], g)
        compare_topk(host(loop.topk), sel["topk_idx"], sel["scores"], g.topk)
        gtopk = host(loop.topk)
        if mass == "token":
            m_o = oracle.token_mass(ch["q"], before["k_p"], before["persist_len"], k_l, gtopk, g)
        else:
            m_o = sel["mass"]
        after = dict(k_p=host(cache.k_pers), v_p=host(cache.v_pers), persist_len=host(cache.persist_len),
                     persist_src=host(cache.persist_src), persist_kbar=host(cache.persist_kbar))
        keep_o, admit_o = oracle.update_decisions(m_o, before["persist_len"], rh, g)
        keep_g, admit_g = decisions_from_state(before, after, s, g.n_qblk)
        tot_heads += compare_update_decisions(keep_g, admit_g, keep_o, admit_o, m_o, before["persist_len"], rh, g)
        moved = oracle.apply_update(before, keep_g, admit_g, k_l, v_l, host(loop.kbar_local), rh, s, g)
        for k in ("k_p", "v_p", "persist_len", "persist_src", "persist_kbar"):
            np.testing.assert_array_equal(after[k], moved[k], err_msg=f"step {s} {k}")
        if s == 0:
            # the first chunk to leave the window fills the sinks with its first frame
            assert (after["persist_src"][..., :nq_frame] == np.arange(nq_frame)).all()
            assert (after["persist_len"] > 0).sum(-1).min() == g.n_qblk
            sink_src = after["persist_src"][..., :nq_frame].copy()
        else:
            np.testing.assert_array_equal(after["persist_src"][..., :nq_frame], sink_src)
    print(f"{mass}: rollout from empty cache, {cfg['steps']} steps, near-tie update heads {tot_heads}, "
          f"final valid slots {(host(cache.persist_len) > 0).sum(-1).tolist()}")
