"""Helpers for the GPU parity tests: host<->device moves and the comparison bars."""
import sys

import numpy as np
import torch

# Output tolerances against the fp64 oracle.
BF16_MAX, BF16_MEAN = 1e-2, 1e-3  # bf16 inputs, fp32 accumulation
F32_MAX = 1e-5  # fp32 path


def bf16_half_ulp(x):
    """Half the spacing of bf16 numbers at |x| (0 at x = 0): the most that storing a
    value of that magnitude in bf16 moves it.  It reaches 7.8e-3 for |x| in [2, 4)
    and 1.6e-2 for |x| in [4, 8)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, e = np.frexp(a)  # a = m * 2**e with m in [0.5, 1): the bf16 spacing there is 2**(e - 8)
    return np.where(a > 0, np.ldexp(1.0, e - 9), 0.0)


def bf16_excess(got, ref):
    """|got - ref| beyond the bf16 rounding of the stored output got: the error the
    fp32 computation made.  The max bar applies to this; the mean bar to |got - ref|."""
    got = np.asarray(got, dtype=np.float64)
    return np.abs(got - ref) - bf16_half_ulp(got)


def check_bf16_outputs(got, ref, what=""):
    """Max and mean bars of bf16 outputs: max of bf16_excess <= 1e-2, mean |got - ref|
    <= 1e-3.  Returns (max |got - ref|, max excess, mean)."""
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    exc = bf16_excess(got, ref)
    mx, mx_exc, mean = float(err.max()), float(exc.max()), float(err.mean())
    assert mx_exc <= BF16_MAX and mean <= BF16_MEAN, (
        f"{what}: max {mx:.3e} (beyond bf16 rounding {mx_exc:.3e}) mean {mean:.3e}")
    return mx, mx_exc, mean


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
        exc = float(bf16_excess(got, ref).max())
        info += f", beyond bf16 rounding {exc:.3e}"
        assert exc <= BF16_MAX and mean <= BF16_MEAN, info
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
