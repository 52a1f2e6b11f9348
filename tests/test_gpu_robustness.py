"""Device-state robustness: a ring head or step counter outside its range,
written from the host, must neither fault nor index out of bounds.  The
kernels reduce the ring head into [0, R) (so results equal those of the
reduced head) and raise sticky bits in the device status word, which
pbsa_device_status reads back and clears.  Every kernel exits normally."""
import numpy as np
import pytest
import torch

import block_sparse_attention_15_amd as pb
from block_sparse_attention_15_amd import _lib
import synth
from pbsa_harness import GpuStep, host
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu


def read_status(clear=True):
    out = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    pb.pbsa_device_status(out, clear)
    torch.cuda.synchronize()
    return int(out.item())


@pytest.mark.parametrize("bad_head", [5, -3, 2 ** 31 - 1, -(2 ** 31)])
def test_corrupt_ring_head_is_reduced_and_flagged(bad_head):
    cfg = SMALL["ragged_bf16"]
    x = synth.make_step_inputs(cfg)
    read_status()                                  # start from a clear word
    R = pb.pbsa_plan(cfg).ring_chunks
    good = ((bad_head % R) + R) % R
    runs = {}
    for head in (good, bad_head):
        st = GpuStep(cfg, x)
        st.ring_head.fill_(head)
        kn = torch.ones_like(st.q)
        pb.pbsa_ring_append(st.p, kn, kn, st.ring_head, st.k_l, st.v_l, st.kbar_l)
        st.score_select()
        st.update(2)
        torch.cuda.synchronize()
        runs[head] = (st, read_status())
    st_g, flag_g = runs[good]
    st_b, flag_b = runs[bad_head]
    assert flag_g == 0
    assert flag_b & _lib.PBSA_DEVICE_BAD_RING_HEAD
    assert read_status() == 0, "the read clears the word"
    for name in ("k_l", "v_l", "topk", "mass", "kbar_l", "k_p", "v_p", "plen", "psrc", "pkbar", "n_rep"):
        assert torch.equal(getattr(st_g, name), getattr(st_b, name)), name
    assert int(host(st_b.ring_head)[0]) == (good + 1) % R


def test_bad_step_counter_is_flagged():
    cfg = SMALL["ragged_bf16"]
    x = synth.make_step_inputs(cfg)
    read_status()
    st = GpuStep(cfg, x)
    st.score_select()
    st.update(-4)
    torch.cuda.synchronize()
    assert read_status() == _lib.PBSA_DEVICE_BAD_STEP_COUNTER
    st = GpuStep(cfg, x)
    st.score_select()
    st.update(3)
    torch.cuda.synchronize()
    assert read_status(clear=False) == 0
    assert read_status() == 0
