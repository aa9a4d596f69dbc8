"""Calibrated block-sparse spatiotemporal attention on AMD MI355X (gfx950).

Python binding of libcalibattn.so (C ABI in include/calibattn.h).  The library is
loaded on first use; a missing library raises instead of falling back.
"""
from .api import (
    CalibAttnError,
    block_energy_from_lse,
    build_block_csr,
    build_block_intervals,
    calib_block_energy,
    calib_block_energy_noalloc,
    calib_block_energy_ws,
    dense_attn_fwd,
    energy_workspace_bytes,
    make_desc,
    n_blocks,
    order_heavy_rows_first,
    rep_row_broadcast,
    select_blocks_by_energy,
    select_blocks_by_energy_heads,
    select_rep_heads,
    sparse_attn_fwd,
    sparse_attn_fwd_intervals,
    spatial_rep_similarity,
    version,
)
from ._lib import LIB_PATH, LibraryMissing, load as load_library

__all__ = [
    "CalibAttnError",
    "LibraryMissing",
    "LIB_PATH",
    "block_energy_from_lse",
    "build_block_csr",
    "build_block_intervals",
    "calib_block_energy",
    "calib_block_energy_noalloc",
    "calib_block_energy_ws",
    "dense_attn_fwd",
    "energy_workspace_bytes",
    "load_library",
    "make_desc",
    "n_blocks",
    "order_heavy_rows_first",
    "rep_row_broadcast",
    "select_blocks_by_energy",
    "select_blocks_by_energy_heads",
    "select_rep_heads",
    "sparse_attn_fwd",
    "sparse_attn_fwd_intervals",
    "spatial_rep_similarity",
    "version",
]
