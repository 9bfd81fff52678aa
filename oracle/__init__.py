"""CPU float64 oracle for exact attention -- test infrastructure only.

Imported by tests/, by the package smoke check and by the benchmark's CPU
baseline leg; never by the GPU library.
"""
from .attention import (  # noqa: F401
    scores, forward, backward, merge, tiled_forward, forward_rows,
    backward_dq_rows, backward_dkdv_rows, probs, forward_kvcache,
    forward_varlen, backward_varlen, block_allowed, forward_blocksparse, backward_blocksparse,
    blocksparse_rows, blocksparse_dkdv_cols,
)
