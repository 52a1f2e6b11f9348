"""The backward captured into a HIP graph and replayed.

`pbsa_bwd` enqueues its preparation and five MFMA kernels on the caller's
stream, which stream capture records in order.  The captured graph is
replayed three times, with the
outputs refilled with NaN (eager work) and a synchronisation between
replays, and every replay must equal the eager call bit for bit (the
backward is deterministic: one owner per output element, fixed order).
"""
import numpy as np
import pytest
import torch

import block_sparse_attention_15_amd as pb
import oracle
import synth
from pbsa_harness import GpuStep, dev, host
from test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["ragged_bf16", "ragged_bf16_d64_b2"])
def test_bwd_graph_replay_equals_eager(name):
    cfg = SMALL[name]
    x = synth.make_step_inputs(cfg)
    g = oracle.geometry(cfg)
    kbar_p = oracle.pool_slots(x["k_p"], x["persist_len"])
    sel = oracle.score_select(x["q"], x["k_l"], 0, kbar_p, x["persist_len"], g)
    st = GpuStep(cfg, x)
    topk = dev(sel["topk_idx"])
    st.fwd(topk)
    dout = dev(synth.make_dout(cfg, seed=cfg["seed"] + 100), st.p.torch_dtype)
    eager = {k: host(v) for k, v in st.bwd(dout, topk).items()}
    torch.cuda.synchronize()

    s = pb.shapes(st.p)
    f = dict(dtype=torch.float32, device="cuda")
    out = dict(dq=torch.empty(s["q"], **f), dk_p=torch.empty(s["k_pers"], **f), dv_p=torch.empty(s["k_pers"], **f),
               dk_l=torch.empty(s["k_local"], **f), dv_l=torch.empty(s["k_local"], **f))
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        pb.pbsa_bwd(st.p, st.q, st.k_p, st.v_p, st.plen, st.k_l, st.v_l, topk, st.o, st.lse, dout, out["dq"],
                    out["dk_p"], out["dv_p"], out["dk_l"], out["dv_l"], st.ws_bwd)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in out.values():
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, t in out.items():
            got = host(t)
            assert np.isfinite(got).all(), (name, rep, k)
            np.testing.assert_array_equal(got, eager[k], err_msg=f"{name} replay {rep} {k}")
