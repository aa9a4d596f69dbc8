"""GPU parity at degenerate sizes, through the C ABI binding, against the fp64 oracle:
sequences shorter than one block (down to a single token), one image row per frame
(every grid row an anchor), an anchor stride beyond the frame height, a batch of two
items sharing one mask, and a text prefix with a repetition head through both skip
list forms.  Bars as elsewhere: bf16 max 1e-2 beyond the output's bf16 rounding / mean 1e-3, fp32 max 1e-5; integer
results bit-exact."""
import numpy as np
import pytest
import torch

import calibrated_block_sparse_calib_amd as cba
import oracle
from tests.gpu_util import assert_close_lse, assert_close_out, log, to_host

pytestmark = pytest.mark.gpu


def _inputs(heads, n, d, dtype, seed, batch=1):
    rng = np.random.default_rng(seed)
    x = [rng.standard_normal((batch, heads, n, d)).astype(np.float32) for _ in range(3)]
    if dtype == "bf16":
        x = [torch.from_numpy(a).to(torch.bfloat16).float().numpy() for a in x]
    return x


def _dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t.to(torch.bfloat16) if dtype == "bf16" else t).cuda()


def _mask(heads, nb, seed, density=0.5):
    m = (np.random.default_rng(seed).random((heads, nb, nb)) < density).astype(np.uint8)
    for h in range(heads):
        np.fill_diagonal(m[h], 1)
    return m


@pytest.mark.parametrize("n,block,d,dtype", [(1, 32, 64, "bf16"), (5, 32, 128, "bf16"), (33, 32, 64, "bf16"),
                                             (1, 128, 128, "bf16"), (77, 128, 128, "bf16"), (5, 64, 64, "f32"),
                                             (40, 32, 128, "f32")])
def test_short_sequences(n, block, d, dtype):
    """Sequences of one token up to a few blocks: sparse, dense and energies."""
    log(f"short sequence n={n} B={block} d={d} {dtype}")
    heads = 2
    q, k, v = _inputs(heads, n, d, dtype, seed=n * 7 + block)
    nb = (n + block - 1) // block
    mask = _mask(heads, nb, seed=n)
    qd, kd, vd = _dev(q, dtype), _dev(k, dtype), _dev(v, dtype)
    row_ptr, col_idx, order = cba.build_block_csr(torch.from_numpy(mask).cuda())
    o, lse = cba.sparse_attn_fwd(qd, kd, vd, row_ptr, col_idx, block=block, work_order=order, return_lse=True)
    od, lsed = cba.dense_attn_fwd(qd, kd, vd, block=block, return_lse=True)
    energy, lse_e, _ = cba.calib_block_energy(qd, kd, None, block=block)
    torch.cuda.synchronize()
    for h in range(heads):
        ref, ref_lse = oracle.sparse_attention(q[0, h], k[0, h], v[0, h], mask[h], block)
        assert_close_out(to_host(o)[0, h], ref, dtype, f"sparse h{h}")
        assert_close_lse(to_host(lse)[0, h], ref_lse, f"sparse h{h}", 1e-3 if dtype == "bf16" else 1e-5)
        refd, refd_lse = oracle.dense_attention(q[0, h], k[0, h], v[0, h])
        assert_close_out(to_host(od)[0, h], refd, dtype, f"dense h{h}")
        assert_close_lse(to_host(lse_e)[0, h], refd_lse, f"energy-pass LSE h{h}", 1e-3 if dtype == "bf16" else 1e-5)
        ref_e = oracle.block_energy(q[0, h], k[0, h], block)
        tol = 1e-4 * block if dtype == "bf16" else 1e-5 * block
        assert np.abs(to_host(energy)[0, h] - ref_e).max() <= tol


@pytest.mark.parametrize("grid,stride", [((3, 1, 40), 4), ((2, 5, 24), 8), ((2, 6, 20), 6)])
def test_repetition_degenerate_grids(grid, stride):
    """One image row per frame (every grid row is an anchor: nothing to broadcast),
    a stride beyond the frame height (one anchor row per frame standing for all the
    others), and a stride equal to the height."""
    log(f"repetition grid={grid} stride={stride}")
    heads, d, block, prefix = 2, 128, 64, 64
    n = prefix + int(np.prod(grid))
    q, k, v = _inputs(heads, n, d, "bf16", seed=stride)
    nb = (n + block - 1) // block
    mask = _mask(heads, nb, seed=stride + 1)
    rep = np.array([0, 1], np.uint8)
    qd, kd, vd = _dev(q, "bf16"), _dev(k, "bf16"), _dev(v, "bf16")
    row_ptr, col_idx, _ = cba.build_block_csr(torch.from_numpy(mask).cuda())
    kw = dict(block=block, rep_heads=rep, anchor_stride=stride, n_prefix=prefix, grid=grid, return_lse=True)
    o, lse = cba.sparse_attn_fwd(qd, kd, vd, row_ptr, col_idx, fuse_broadcast=True, **kw)
    o2, _ = cba.sparse_attn_fwd(qd, kd, vd, row_ptr, col_idx, fuse_broadcast=False, o=torch.zeros_like(qd), **kw)
    cba.rep_row_broadcast(o2, rep, stride, block=block, n_prefix=prefix, grid=grid)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    for h in range(heads):
        ref, ref_lse = oracle.sparse_attention_with_repetition(q[0, h], k[0, h], v[0, h], mask[h], block, prefix,
                                                               grid, stride, bool(rep[h]))
        assert_close_out(to_host(o)[0, h], ref, "bf16", f"rep grid h{h}")
        assert_close_lse(to_host(lse)[0, h], ref_lse, f"rep grid h{h}", 1e-3)
    if grid[1] >= 2:
        _, lse_d = cba.dense_attn_fwd(qd, kd, vd, block=block, return_lse=True)
        hs, tc = cba.spatial_rep_similarity(qd, kd, lse_d, stride, n_prefix=prefix, grid=grid)
        torch.cuda.synchronize()
        for h in range(heads):
            toks, cos = oracle.repetition_cosines(q[0, h], k[0, h], prefix, grid, stride)
            assert np.abs(to_host(tc)[0, h][toks] - cos).max() <= 1e-4
            assert abs(float(to_host(hs)[0, h]) - cos.mean()) <= 1e-5


def test_batch_of_two_shares_the_mask():
    """batch = 2: both items use the same per-head mask; each item's outputs match the
    oracle, and the calibration energies are per item (the batch index is the draw)."""
    heads, n, d, block = 3, 300, 64, 64
    q, k, v = _inputs(heads, n, d, "bf16", seed=99, batch=2)
    nb = (n + block - 1) // block
    mask = _mask(heads, nb, seed=98, density=0.4)
    qd, kd, vd = _dev(q, "bf16"), _dev(k, "bf16"), _dev(v, "bf16")
    row_ptr, col_idx, order = cba.build_block_csr(torch.from_numpy(mask).cuda())
    iv_ptr, ivs = cba.build_block_intervals(torch.from_numpy(mask).cuda())
    o = cba.sparse_attn_fwd(qd, kd, vd, row_ptr, col_idx, block=block, work_order=order)
    o_iv = cba.sparse_attn_fwd_intervals(qd, kd, vd, iv_ptr, ivs, block=block)
    energy, _, _ = cba.calib_block_energy(qd, kd, None, block=block)
    torch.cuda.synchronize()
    assert torch.equal(o, o_iv)
    for b in range(2):
        for h in range(heads):
            ref, _ = oracle.sparse_attention(q[b, h], k[b, h], v[b, h], mask[h], block)
            assert_close_out(to_host(o)[b, h], ref, "bf16", f"batch {b} h{h}")
            ref_e = oracle.block_energy(q[b, h], k[b, h], block)
            assert np.abs(to_host(energy)[b, h] - ref_e).max() <= 1e-4 * block
