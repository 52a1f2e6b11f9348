"""CPU oracle for Persistent Block-Sparse Attention (PBSA).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no code
with the HIP library and never imports it.

Source: "Sparse Forcing: Native Trainable Sparse Attention for Real-time
Autoregressive Diffusion Video Generation" -- the abstract (review page and
the OpenAlex / thelatestinai copies), the project page's feature list and its
``SparseForcingAttention`` usage example, and the fragment of the paper's
training algorithm (the cache pass "apply PBSA with top-K and update P and L").

The pages give no equations for block scoring, selection or the persistent
update; every such step follows an explicit reading, listed in ``READINGS``
and restated in each function's docstring.

Precision: attention outputs and gradients are computed in float64.  The
quantities that decide integers (pooled block scores for top-k selection and
pooled masses for the update) are computed in float32, the precision in which
the HIP kernels take the same decisions; token-exact masses are accumulated
in float64 and rounded to float32 before the update ranks them.

Parity pins: every function here is pinned by ``tests/test_oracle_*.py``
(brute force, dense-attention reduction, invariants, closed forms, finite
differences).  No function is "parity unpinned".
"""
from .pbsa import (  # noqa: F401
    READINGS,
    EMPTY_SRC,
    Geometry,
    geometry,
    pool_query_blocks,
    pool_local_blocks,
    pool_slots,
    block_scores,
    select_topk,
    pooled_mass,
    score_select,
    attend,
    attend_bwd,
    token_mass,
    persist_update,
    update_decisions,
    apply_update,
    near_tie_rows,
    ring_append,
    decode_chunk,
)
