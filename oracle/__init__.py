"""CPU fp64 oracle for calibrated block-sparse attention -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The GPU library never calls it and shares no code with it.
"""
from .calibattn_oracle import (
    dense_attention,
    block_energy,
    block_energy_from_lse,
    select_row,
    select_blocks,
    aggregate_votes,
    build_csr,
    build_intervals,
    heavy_first_order,
    computed_rows,
    sparse_attention,
    row_broadcast,
    sparse_attention_with_repetition,
    token_mask_from_blocks,
    repetition_cosines,
    repetition_score,
    mark_repetition_heads,
)

__all__ = [
    "dense_attention",
    "block_energy",
    "block_energy_from_lse",
    "select_row",
    "select_blocks",
    "aggregate_votes",
    "build_csr",
    "build_intervals",
    "heavy_first_order",
    "computed_rows",
    "sparse_attention",
    "row_broadcast",
    "sparse_attention_with_repetition",
    "token_mask_from_blocks",
    "repetition_cosines",
    "repetition_score",
    "mark_repetition_heads",
]
