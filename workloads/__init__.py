"""Seeded synthetic inputs for calibrated block-sparse video attention.

This package produces token grids, Q/K/V tensors and block masks of the shapes of
the video diffusion transformers that the CalibAtt summaries evaluate on
(Wan 2.1 1.3B/14B, Mochi 1, HunyuanVideo).  It holds none of the attention
method's arithmetic: it draws random numbers and lays them out.  Both the GPU
path and the CPU oracle receive the arrays it returns, unchanged.
"""
from .configs import CONFIGS, AttnConfig, get_config
from .generator import (
    grid_coords,
    make_qkv,
    random_block_mask,
    rep_head_flags,
    head_densities,
    to_bf16_array,
)

__all__ = [
    "CONFIGS",
    "AttnConfig",
    "get_config",
    "grid_coords",
    "make_qkv",
    "random_block_mask",
    "rep_head_flags",
    "head_densities",
    "to_bf16_array",
]
