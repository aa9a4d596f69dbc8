"""GPU parity with Q, K and V given as views into larger buffers whose rows past
each head's last token hold NaN.  The kernels stage K and V tiles whose last rows
lie past the end of the sequence; those rows must never reach the arithmetic (a
NaN V row times a zero weight is NaN).  Sequence lengths are chosen with
n % 64 != 0, and with n % B in [1, 64] so that the last key block's second
64-key step lies wholly past the end.  Every output must be finite and within
the usual bars of the fp64 oracle."""
import numpy as np
import pytest
import torch

import calibrated_block_sparse_calib_amd as cba
import oracle
from tests.gpu_util import assert_close_lse, assert_close_out, log, to_host

pytestmark = pytest.mark.gpu

EXTRA_ROWS = 72  # NaN rows after each head's last token (more than one 64-key step)


def _inputs(heads, n, d, dtype, seed):
    rng = np.random.default_rng(seed)
    x = [rng.standard_normal((1, heads, n, d)).astype(np.float32) for _ in range(3)]
    if dtype == "bf16":
        x = [torch.from_numpy(a).to(torch.bfloat16).float().numpy() for a in x]
    return x


def _nan_tail_view(a, dtype, fill=float("nan")):
    """Device view [1, heads, n, d] of a [1, heads, n + EXTRA_ROWS, d] buffer whose
    extra rows hold `fill`."""
    b, h, n, d = a.shape
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    buf = torch.full((b, h, n + EXTRA_ROWS, d), fill, dtype=tdt, device="cuda")
    buf[:, :, :n] = torch.from_numpy(np.ascontiguousarray(a)).to(tdt).cuda()
    return buf[:, :, :n]


@pytest.mark.parametrize("n,block,d,dtype", [
    (424, 128, 128, "bf16"),  # n % 128 = 40: the last block's second 64-key step is empty
    (300, 128, 64, "bf16"),   # n % 128 = 44
    (337, 64, 128, "bf16"),   # n % 64 = 17
    (203, 32, 128, "bf16"),   # n % 32 = 11
    (424, 128, 128, "f32"),
])
def test_nan_rows_past_the_end_never_reach_the_outputs(n, block, d, dtype):
    log(f"NaN tail n={n} B={block} d={d} {dtype}")
    heads = 2
    q, k, v = _inputs(heads, n, d, dtype, seed=n + block)
    qd, kd, vd = (_nan_tail_view(x, dtype) for x in (q, k, v))
    assert qd.stride(1) == (n + EXTRA_ROWS) * d
    nb = (n + block - 1) // block
    rng = np.random.default_rng(n)
    mask = (rng.random((heads, nb, nb)) < 0.6).astype(np.uint8)
    for h in range(heads):
        np.fill_diagonal(mask[h], 1)
    mask[:, :, nb - 1] = 1  # every row keeps the ragged last key block
    row_ptr, col_idx, order = cba.build_block_csr(torch.from_numpy(mask).cuda())
    out = lambda: _nan_tail_view(np.zeros((1, heads, n, d), np.float32), dtype, fill=0.0)
    o, lse = cba.sparse_attn_fwd(qd, kd, vd, row_ptr, col_idx, block=block, work_order=order, o=out(),
                                 return_lse=True)
    od, lsed = cba.dense_attn_fwd(qd, kd, vd, block=block, o=out(), return_lse=True)
    energy, lse_e, oe = cba.calib_block_energy(qd, kd, vd, block=block, o=out())
    results = [("sparse O", o), ("sparse LSE", lse), ("dense O", od), ("dense LSE", lsed),
               ("energy", energy), ("energy-pass LSE", lse_e), ("energy-pass O", oe)]
    if dtype == "bf16":
        e1, l1, o1 = cba.calib_block_energy_ws(qd, kd, vd, block=block, o=out())
        results += [("one-pass energy", e1), ("one-pass LSE", l1), ("one-pass O", o1)]
    torch.cuda.synchronize()
    for name, t in results:
        assert torch.isfinite(t).all(), f"{name}: non-finite values"
    tol_lse = 1e-3 if dtype == "bf16" else 1e-5
    etol = 1e-4 * block if dtype == "bf16" else 1e-5 * block
    for h in range(heads):
        ref, ref_lse = oracle.sparse_attention(q[0, h], k[0, h], v[0, h], mask[h], block)
        assert_close_out(to_host(o)[0, h], ref, dtype, f"sparse h{h}")
        assert_close_lse(to_host(lse)[0, h], ref_lse, f"sparse h{h}", tol_lse)
        refd, refd_lse = oracle.dense_attention(q[0, h], k[0, h], v[0, h])
        assert_close_out(to_host(od)[0, h], refd, dtype, f"dense h{h}")
        assert_close_out(to_host(oe)[0, h], refd, dtype, f"energy-pass O h{h}")
        assert_close_lse(to_host(lse_e)[0, h], refd_lse, f"energy-pass LSE h{h}", tol_lse)
        ref_e = oracle.block_energy(q[0, h], k[0, h], block)
        assert np.abs(to_host(energy)[0, h] - ref_e).max() <= etol
        if dtype == "bf16":
            assert np.abs(to_host(e1)[0, h] - ref_e).max() <= etol
            assert_close_out(to_host(o1)[0, h], refd, dtype, f"one-pass O h{h}")


def test_nan_tail_repetition_similarity():
    """spatial_rep_similarity over K with NaN rows past the end (ragged last step)."""
    heads, d, prefix, grid, stride = 2, 128, 32, (2, 6, 25), 3
    n = prefix + int(np.prod(grid))  # 332: n % 64 = 12
    q, k, v = _inputs(heads, n, d, "bf16", seed=5)
    qd, kd, vd = (_nan_tail_view(x, "bf16") for x in (q, k, v))
    _, lse = cba.dense_attn_fwd(qd, kd, vd, block=64, o=_nan_tail_view(np.zeros_like(q), "bf16", 0.0),
                                return_lse=True)
    hs, tc = cba.spatial_rep_similarity(qd, kd, lse, stride, n_prefix=prefix, grid=grid)
    torch.cuda.synchronize()
    assert torch.isfinite(hs).all()
    for h in range(heads):
        toks, cos = oracle.repetition_cosines(q[0, h], k[0, h], prefix, grid, stride)
        got = to_host(tc)[0, h][toks]
        assert np.isfinite(got).all()
        assert np.abs(got - cos).max() <= 1e-4
