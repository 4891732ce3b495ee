"""fp64 CPU oracle for the masked, biased triangle-attention forward and its
gradient.

TEST INFRASTRUCTURE ONLY: the checker that the GPU library is compared
against.  Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import this package.  It shares no code with the HIP
library and never imports it.
"""
from .oracle import (  # noqa: F401
    MASK_BLOCK,
    MASK_DENSE,
    MASK_KV_LENGTHS,
    MASK_NONE,
    MOD_CAUSAL,
    MOD_NONE,
    OracleBlockMask,
    build,
    build_bwd,
    default_threads,
    load_library,
    oracle_bwd,
    oracle_fwd,
)
