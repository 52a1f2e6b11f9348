"""The allocation-free scoring entry point (pbsa_score_select_noalloc, scratch
in a static device array of the library) against pbsa_score_select with a
caller workspace: the same selections and masses, bit for bit, on two calls
in a row -- the decode shape, then a smaller one that reuses the same array
-- and a configuration too large for the array is rejected before launch."""
import pytest
import torch

import block_sparse_attention_15_amd as pb
from block_sparse_attention_15_amd import _lib
import synth
from pbsa_harness import GpuStep

pytestmark = pytest.mark.gpu


def small_cfg():
    return dict(batch=1, heads=2, head_dim=128, frame_h=14, frame_w=22, block_t=1, block_h=8, block_w=8,
                chunk_frames=2, total_cache_size=7 * 308, local_cache_size=4 * 308, persistent_cache_size=3 * 308,
                use_local_block_sparse_attn=1, topk_ratio=0.25, softmax_scale=0.0, dtype="bf16", seed=81,
                plant_frac=0.1, alpha=4.0)


def run_both(cfg, ring_head):
    x = synth.make_step_inputs(cfg)
    x["ring_head"][:] = ring_head
    st = GpuStep(cfg, x)
    st.score_select()
    topk = torch.full_like(st.topk, -7)
    mass = torch.full_like(st.mass, float("nan"))
    pb.pbsa_score_select_noalloc(st.p, st.q, st.kbar_l, st.ring_head, st.pkbar, st.plen, topk, mass)
    torch.cuda.synchronize()
    return st, topk, mass


def test_noalloc_equals_workspace_entry_twice():
    for cfg, rh in ((synth.workload("decode_c1"), 1), (small_cfg(), 0)):
        st, topk, mass = run_both(cfg, rh)
        assert torch.equal(topk, st.topk), cfg["frame_h"]
        assert torch.equal(mass, st.mass), cfg["frame_h"]


def test_noalloc_rejects_configs_beyond_its_scratch():
    big = dict(synth.workload("decode_c1"), batch=64)  # 11.4 MB of column sums (eight query blocks per workgroup)
    p = pb.pbsa_plan(big)
    assert p.ws_score_select > 8 << 20
    lib = _lib.load()
    c = pb.make_config(big)
    import ctypes
    st = lib.pbsa_score_select_noalloc(ctypes.byref(c), *(ctypes.c_void_p(0x1000 * (i + 1)) for i in range(7)), None)
    assert st == _lib.PBSA_ERR_WORKSPACE
    assert b"static array" in lib.pbsa_last_error()
