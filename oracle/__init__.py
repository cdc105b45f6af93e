"""fp64 CPU oracle for mean-corrected block-sparse causal prefill.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The product path (the HIP library
and its Python binding) never imports, calls or links it, and it shares no
code with that path.
"""
from .oracle import (  # noqa: F401
    block_bounds,
    pool_keys,
    pool_queries,
    select_blocks,
    forced_keep,
    attend,
    attend_row,
    attend_loop,
    prefill,
    gather_paged,
    csr_from_sets,
    OracleResult,
)
