"""Seeded synthetic inputs for block-sparse causal prefill.

This package creates inputs only. It holds none of the attention method's
arithmetic: no pooling, no scoring, no softmax. Both the fp64 oracle's tests
and the GPU path's tests and benchmark draw their inputs from here, so that
the two sides see the same bytes.
"""
from .generators import (  # noqa: F401
    CONFIGS,
    Workload,
    chunk_of,
    make_workload,
    planted_prefill,
    fp8_e4m3_encode,
    fp8_e4m3_decode,
    quantize_fp8_per_tensor,
    to_bf16,
    paginate,
)
