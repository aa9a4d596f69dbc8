"""Seeded input generator (NumPy).  Random draws and layout only.

Recipe for the video workloads:
  * grid positions p = (f / lt, y / ls, x / ls) for every grid token;
  * a random-Fourier positional feature phi(p) in R^d with components
    sqrt(2) * cos(w_k . p + b_k), w_k ~ N(0, I_3), b_k ~ U[0, 2 pi); its seed
    depends on the head (and timestep bucket) only, so it is the same in every
    draw -- the input-independent structure the calibration is meant to find;
  * Q = N(0,1) + amp * phi and K = N(0,1) + amp * phi (same phi: 3-D locality),
    V = N(0,1); the noise seed depends on (draw, head, tensor);
  * non-grid (text) tokens get plain N(0,1) rows;
  * bf16 workloads are rounded to bf16 once (round to nearest even) and every
    consumer sees the rounded values.

Every random stream is keyed by a SeedSequence built from
(config seed, role, bucket, draw, head), so any head of any draw can be
regenerated alone and in any order.
"""
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

from .configs import AttnConfig

ROLE_PHI, ROLE_Q, ROLE_K, ROLE_V, ROLE_MASK, ROLE_REP, ROLE_LS, ROLE_DENS = range(1, 9)


def _rng(cfg: AttnConfig, role: int, bucket: int = 0, draw: int = 0, head: int = 0):
    ss = np.random.SeedSequence([int(cfg.seed), role, bucket, draw, head])
    return np.random.Generator(np.random.PCG64(ss))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def grid_coords(cfg: AttnConfig):
    """(f, y, x) integer coordinates of the grid tokens, in frame-major order."""
    f_, h_, w_ = cfg.grid
    t = np.arange(cfg.n_grid, dtype=np.int64)
    return t // (h_ * w_), (t // w_) % h_, t % w_


def to_bf16_array(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32
    holding bf16-representable values.  Finite inputs only."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def head_ls_scale(cfg: AttnConfig) -> np.ndarray:
    """Per-head multiplier of the spatial and temporal length scales
    (log-uniform over cfg.ls_log_range; 1 when unset)."""
    if cfg.ls_log_range is None:
        return np.ones(cfg.heads)
    lo, hi = cfg.ls_log_range
    rng = _rng(cfg, ROLE_LS)
    return np.exp(rng.uniform(np.log(lo), np.log(hi), size=cfg.heads))


def phi_features(cfg: AttnConfig, head: int, bucket: int = 0) -> np.ndarray:
    """Positional feature [seq_len, d] (float32); zero rows for text tokens."""
    d = cfg.head_dim
    out = np.zeros((cfg.seq_len, d), dtype=np.float32)
    if cfg.phi_amp == 0.0:
        return out
    rng = _rng(cfg, ROLE_PHI, bucket, 0, head)
    omega = rng.standard_normal((d, 3))
    beta = rng.uniform(0.0, 2.0 * np.pi, size=d)
    scale = head_ls_scale(cfg)[head] * cfg.bucket_ls_scale[bucket % len(cfg.bucket_ls_scale)]
    f, y, x = grid_coords(cfg)
    pos = np.stack([f / (cfg.lt * scale), y / (cfg.ls * scale), x / (cfg.ls * scale)], axis=1)
    arg = pos @ omega.T + beta
    out[cfg.n_prefix:] = (np.sqrt(2.0) * np.cos(arg)).astype(np.float32)
    return out


def _one_head(cfg, draw, head, bucket, with_v):
    n, d = cfg.seq_len, cfg.head_dim
    phi = phi_features(cfg, head, bucket)
    amp = np.float32(cfg.phi_amp)
    q = _rng(cfg, ROLE_Q, bucket, draw, head).standard_normal((n, d), dtype=np.float32)
    q += amp * phi
    k = _rng(cfg, ROLE_K, bucket, draw, head).standard_normal((n, d), dtype=np.float32)
    k += amp * phi
    v = None
    if with_v:
        v = _rng(cfg, ROLE_V, bucket, draw, head).standard_normal((n, d), dtype=np.float32)
    if cfg.dtype == "bf16":
        q, k = to_bf16_array(q), to_bf16_array(k)
        if v is not None:
            v = to_bf16_array(v)
    return q, k, v


def make_qkv(cfg: AttnConfig, draw: int, heads=None, bucket: int = 0, with_v: bool = True):
    """Q, K, V as float32 arrays [len(heads), seq_len, d] (bf16-representable for
    bf16 workloads).  `draw` selects the noise; draws 0..calib_draws-1 are the
    calibration draws and draw == calib_draws is the held-out evaluation input."""
    if heads is None:
        heads = range(cfg.heads)
    heads = list(heads)
    n, d = cfg.seq_len, cfg.head_dim
    q = np.empty((len(heads), n, d), dtype=np.float32)
    k = np.empty_like(q)
    v = np.empty_like(q) if with_v else None

    def work(i):
        qi, ki, vi = _one_head(cfg, draw, heads[i], bucket, with_v)
        q[i], k[i] = qi, ki
        if with_v:
            v[i] = vi

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(len(heads))))
    return q, k, v


def head_densities(cfg: AttnConfig) -> np.ndarray:
    """Per-head target density of a Bernoulli mask, uniform over density_range."""
    lo, hi = cfg.density_range
    return _rng(cfg, ROLE_DENS).uniform(lo, hi, size=cfg.heads)


def random_block_mask(cfg: AttnConfig, force_diag: bool = True) -> np.ndarray:
    """Seeded Bernoulli block mask uint8 [heads, nb, nb] (1 = kept) with the
    per-head density from head_densities; the diagonal is set when force_diag."""
    nb = cfg.nb
    dens = head_densities(cfg)
    m = np.empty((cfg.heads, nb, nb), dtype=np.uint8)
    for h in range(cfg.heads):
        m[h] = (_rng(cfg, ROLE_MASK, 0, 0, h).random((nb, nb)) < dens[h]).astype(np.uint8)
        if force_diag:
            np.fill_diagonal(m[h], 1)
    return m


def rep_head_flags(cfg: AttnConfig) -> np.ndarray:
    """uint8 [heads]: 1 for the spatial-repetition heads of the workload."""
    flags = np.zeros(cfg.heads, dtype=np.uint8)
    if cfg.rep_heads_fixed:
        flags[list(cfg.rep_heads_fixed)] = 1
    elif cfg.n_rep_heads:
        idx = _rng(cfg, ROLE_REP).choice(cfg.heads, size=cfg.n_rep_heads, replace=False)
        flags[idx] = 1
    return flags
