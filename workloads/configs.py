"""The five synthetic workloads: token grids of the video models the CalibAtt
summaries evaluate on, plus a tiny grid the CPU oracle checks in full.

Token order is frame-major: token t = n_prefix + f*H*W + y*W + x for a grid
token, and the n_prefix non-grid (text) tokens come first.

Length scales (lt, ls) set how far the smooth positional structure of Q and K
reaches in frames and in pixels; they were tuned once so that calibration at
tau = 0.95 gives the stated mean block densities, and are fixed here.
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class AttnConfig:
    name: str
    heads: int
    head_dim: int
    grid: Tuple[int, int, int]  # (F, H, W)
    block: int
    dtype: str  # "f32" or "bf16"
    seed: int
    n_prefix: int = 0
    phi_amp: float = 2.0  # amplitude of the positional feature in Q and K
    lt: float = 1.0  # temporal length scale (frames)
    ls: float = 1.0  # spatial length scale (pixels)
    ls_log_range: Optional[Tuple[float, float]] = None  # per-head ls multiplier, log-uniform
    mask_mode: str = "calibrate"  # "calibrate" or "bernoulli"
    calib_draws: int = 4
    tau: float = 0.95
    rho: float = 0.5
    density_range: Tuple[float, float] = (0.4, 0.4)  # bernoulli masks: per-head density range
    n_rep_heads: int = 0
    rep_heads_fixed: Tuple[int, ...] = ()
    anchor_stride: int = 4
    buckets: int = 1
    bucket_ls_scale: Tuple[float, ...] = (1.0,)
    notes: str = ""

    @property
    def n_grid(self) -> int:
        f, h, w = self.grid
        return f * h * w

    @property
    def seq_len(self) -> int:
        return self.n_prefix + self.n_grid

    @property
    def nb(self) -> int:
        return (self.seq_len + self.block - 1) // self.block

    @property
    def n_prefix_blocks(self) -> int:
        return self.n_prefix // self.block


CONFIGS = {
    "tiny": AttnConfig(
        name="tiny",
        heads=2,
        head_dim=64,
        grid=(4, 8, 8),
        block=32,
        dtype="f32",
        seed=0,
        phi_amp=0.0,
        mask_mode="calibrate",
        calib_draws=3,
        tau=0.9,
        density_range=(0.4, 0.4),
        rep_heads_fixed=(1,),
        anchor_stride=4,
        notes="plain N(0,1) Q/K/V; calibration (3 draws, tau 0.9) and a 40% Bernoulli mask",
    ),
    "wan13_480p": AttnConfig(
        name="wan13_480p",
        heads=12,
        head_dim=128,
        grid=(21, 30, 52),
        block=128,
        dtype="bf16",
        seed=1,
        lt=15.86,
        ls=37.0,
        mask_mode="calibrate",
        calib_draws=4,
        tau=0.95,
        notes="Wan-2.1-1.3B 480p shape; calibrated masks, ~30% mean density",
    ),
    "wan14_720p": AttnConfig(
        name="wan14_720p",
        heads=40,
        head_dim=128,
        grid=(21, 45, 80),
        block=128,
        dtype="bf16",
        seed=2,
        lt=15.86,
        ls=37.0,
        mask_mode="bernoulli",
        density_range=(0.2, 0.5),
        n_rep_heads=10,
        anchor_stride=4,
        notes="Wan-2.1-14B 720p shape; seeded per-head masks, 10 repetition heads",
    ),
    "mochi": AttnConfig(
        name="mochi",
        heads=24,
        head_dim=128,
        grid=(28, 30, 53),
        block=128,
        dtype="bf16",
        seed=3,
        n_prefix=256,
        lt=15.86,
        ls=37.0,
        mask_mode="calibrate",
        calib_draws=4,
        tau=0.95,
        buckets=3,
        bucket_ls_scale=(0.7, 1.0, 1.4),
        notes="Mochi-1 joint attention: 256 dense text tokens first; 3 timestep buckets",
    ),
    "hunyuan": AttnConfig(
        name="hunyuan",
        heads=24,
        head_dim=128,
        grid=(33, 45, 80),
        block=128,
        dtype="bf16",
        seed=4,
        lt=24.86,
        ls=58.0,
        ls_log_range=(0.5, 2.1),
        mask_mode="calibrate",
        calib_draws=4,
        tau=0.95,
        notes="HunyuanVideo 8 s 720p shape; head-adaptive density 10-60%",
    ),
}

# Positional names for the five workloads, in the order they are usually listed.
CONFIG_ORDER = ("tiny", "wan13_480p", "wan14_720p", "mochi", "hunyuan")


def get_config(name_or_index) -> AttnConfig:
    if isinstance(name_or_index, int):
        return CONFIGS[CONFIG_ORDER[name_or_index]]
    return CONFIGS[name_or_index]
