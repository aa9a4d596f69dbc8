"""Helpers for the GPU parity tests: host<->device moves and the comparison bars."""
import sys

import numpy as np
import torch

# Output tolerances against the fp64 oracle.
BF16_MAX, BF16_MEAN = 1e-2, 1e-3  # bf16 inputs, fp32 accumulation
F32_MAX = 1e-5  # fp32 path


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    """[heads, N, d] float32 host array -> [1, heads, N, d] device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(x))[None]
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.cuda()


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def assert_close_out(got: np.ndarray, ref: np.ndarray, dtype: str, what: str, rows=None):
    if rows is not None:
        got, ref = got[rows], ref[rows]
    err = np.abs(got.astype(np.float64) - ref)
    mx, mean = float(err.max()), float(err.mean())
    at = np.unravel_index(int(np.argmax(err)), err.shape)
    info = f"{what}: max {mx:.3e} at {at} (ref {float(ref[at]):.4f}, got {float(got[at]):.4f}) mean {mean:.3e}"
    if dtype == "bf16":
        assert mx <= BF16_MAX and mean <= BF16_MEAN, info
    else:
        assert mx <= F32_MAX, info
    log("  ok " + info)
    return mx, mean


def assert_close_lse(got: np.ndarray, ref: np.ndarray, what: str, tol: float):
    fin = np.isfinite(ref)
    assert (np.isfinite(got) == fin).all(), f"{what}: -inf pattern differs"
    if fin.any():
        err = float(np.abs(got[fin] - ref[fin]).max())
        assert err <= tol, f"{what}: lse max err {err:.3e}"
