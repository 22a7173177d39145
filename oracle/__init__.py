"""CPU oracle for exact scaled-dot-product attention (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The HIP library never calls it and shares no code with it.
"""
from .attention import (  # noqa: F401
    forward,
    forward_head,
    forward_rows,
    backward,
    backward_head,
    backward_dq_rows,
    backward_kv_cols,
    forward_key_blocked,
    forward_query_chunked,
    forward_scalar,
)
