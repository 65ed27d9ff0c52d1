"""CPU oracle for the CSA / HCA hot path (fp64, numpy).

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import anything under oracle/.  The product path never
routes through it.  Shares no code with the HIP library.
"""
from .csa import (  # noqa: F401
    attend,
    compress,
    csa_entries,
    csa_layer,
    csa_sparse_attn,
    hca_attn,
    index_query,
    index_scores,
    latent_output,
    latent_query,
    merge_weights,
    topk,
    topk_row,
    visible_blocks,
    window_positions,
)
from . import formats  # noqa: F401
