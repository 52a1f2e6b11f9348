"""Persistent Block-Sparse Attention (PBSA) for AMD Instinct MI355X (gfx950).

A thin Python binding over the C ABI of ``libpbsa.so`` (declared in
``include/pbsa.h``).  Every step of the method runs in hand-written HIP
kernels; importing the API requires the built library and fails loudly when
it is missing.
"""
from .api import (  # noqa: F401
    Plan,
    PbsaError,
    make_config,
    pbsa_plan,
    pbsa_pool_slots,
    pbsa_pool_local,
    pbsa_score_select,
    pbsa_score_select_noalloc,
    pbsa_fwd,
    pbsa_fwd_mass,
    pbsa_bwd,
    pbsa_persist_update,
    pbsa_ring_append,
    pbsa_device_status,
    shapes,
    workspace,
)
from .module import PBSACache, SparseForcingAttention  # noqa: F401
from . import _lib

LIB_PATH = _lib.LIB_PATH


def load_library():
    """Load libpbsa.so (raises ImportError if it has not been built)."""
    return _lib.load()
