"""The LDS-race check build (libpbsa_ldscheck.so: the same sources with every
LDS-bound load waited for at once and every step barrier draining all loads
in flight) against the product library, bit for bit: scoring, top-k and
masses, the forward, the token-mass forward, all five gradients and the
persistent update, on shapes that take every LDS-staged path (packed and
per-slot persistent kernels, LDS and global-memory row lookups of the local
kernels, head_dim 64 and 128, [3,4,4] blocks) and on the decode shape.  A
kernel whose waves read a step buffer before its rows land, or load rows into
a buffer that another wave still reads, gives different bits in one of the
two builds."""
import contextlib
import os

import pytest
import torch

import block_sparse_attention_15_amd as pb
from block_sparse_attention_15_amd import _lib
from block_sparse_attention_15_amd.build import LIB_LDS_CHECK
import synth
from pbsa_harness import GpuStep
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu


@contextlib.contextmanager
def check_library():
    """Route the binding's calls to the check library for the block."""
    if not os.path.exists(LIB_LDS_CHECK):
        raise ImportError(f"{LIB_LDS_CHECK} not built (python -m block_sparse_attention_15_amd.build --lds-check)")
    product = _lib.load()
    _lib._lib = None
    try:
        _lib.load(LIB_LDS_CHECK)
        yield
    finally:
        _lib._lib = product


def run_all(cfg, x, dout):
    st = GpuStep(cfg, x)
    st.score_select()
    st.fwd()
    out = dict(topk=st.topk.clone(), mass=st.mass.clone(), o=st.o.clone(), lse=st.lse.clone())
    out.update(st.bwd(dout))
    st.fwd_mass()
    out.update(o_mass=st.o.clone(), lse_mass=st.lse.clone(), token_mass=st.mass.clone())
    st.mass.copy_(out["mass"])
    st.update(0)
    out.update(k_p=st.k_p, v_p=st.v_p, plen=st.plen, psrc=st.psrc, pkbar=st.pkbar, n_rep=st.n_rep,
               ring_head=st.ring_head)
    torch.cuda.synchronize()
    return out


CASES = ["ragged_bf16", "ragged_bf16_d64_b2", "dense_local_huge_bf16", "block344_bf16", "big_persistent_bf16",
         "tiny_bf16", "decode_c1"]


@pytest.mark.parametrize("name", CASES)
def test_check_build_equals_product_build(name):
    cfg = synth.workload("decode_c1") if name == "decode_c1" else SMALL[name]
    x = synth.make_step_inputs(cfg)
    p = pb.pbsa_plan(cfg)
    dout = torch.from_numpy(synth.make_dout(cfg, seed=cfg["seed"] + 100)).to(p.torch_dtype).cuda()
    ref = run_all(cfg, x, dout)
    with check_library():
        got = run_all(cfg, x, dout)
    for k, v in ref.items():
        assert torch.equal(v, got[k]), (name, k)
