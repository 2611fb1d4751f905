"""fp64 CPU oracle for blockwise ring attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call, link
or execute this package: only the test suite, the smoke check and the
benchmark's CPU-baseline leg use it. It shares no code with the HIP library.
"""
from .attention import (  # noqa: F401
    attention,
    attention_rows,
    decode,
    host_positions,
    lse_merge,
    step_partial,
    pair_counts,
)
from .backward import attention_bwd, attention_bwd_sampled  # noqa: F401
