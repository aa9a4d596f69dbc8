"""Seeded random shapes through every call, against the fp64 oracle: head_dim,
block, token grid, text prefix, anchor stride, mask density, dtype and batch drawn
from a fixed seed per case, so that corners no hand-picked case covers get
exercised.  Bars as elsewhere: bf16 max 1e-2 beyond the output's bf16 rounding /
mean 1e-3, fp32 max 1e-5, energies
1e-4 * block (1e-5 * block in fp32), repetition cosines 1e-4 (1e-5 in fp32),
integer results bit-exact."""
import os

import numpy as np
import pytest
import torch

import calibrated_block_sparse_calib_amd as cba
import oracle
from tests.gpu_util import assert_close_out, log, to_host

pytestmark = pytest.mark.gpu

N_CASES = int(os.environ.get("CBA_RANDOM_CASES", "24"))  # more cases for an occasional wider sweep


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    d = int(rng.choice([64, 128]))
    block = int(rng.choice([32, 64, 128]))
    dtype = "f32" if rng.random() < 0.25 else "bf16"
    grid = (int(rng.integers(1, 4)), int(rng.integers(1, 10)), int(rng.integers(1, 30)))
    n_prefix = block * int(rng.integers(0, 3))
    if n_prefix + int(np.prod(grid)) > 700:
        grid = (1, grid[1], max(1, 700 // max(grid[1], 1) // 2))
    stride = int(rng.integers(1, 6))
    heads = int(rng.integers(1, 4))
    batch = int(rng.integers(1, 3))
    density = float(rng.uniform(0.1, 0.9))
    return dict(d=d, block=block, dtype=dtype, grid=grid, n_prefix=n_prefix, stride=stride, heads=heads,
                batch=batch, density=density, rng=rng)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_shape(seed):
    c = _case(seed)
    rng = c.pop("rng")
    d, block, dtype, grid, n_prefix = c["d"], c["block"], c["dtype"], c["grid"], c["n_prefix"]
    stride, heads, batch = c["stride"], c["heads"], c["batch"]
    n = n_prefix + int(np.prod(grid))
    nb = (n + block - 1) // block
    log(f"case {seed}: {c} n={n}")
    x = [rng.standard_normal((batch, heads, n, d)).astype(np.float32) for _ in range(3)]
    if dtype == "bf16":
        x = [torch.from_numpy(a).to(torch.bfloat16).float().numpy() for a in x]
    q, k, v = x
    dev = lambda a: (torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16) if dtype == "bf16"
                     else torch.from_numpy(np.ascontiguousarray(a))).cuda()
    qd, kd, vd = dev(q), dev(k), dev(v)
    mask = (rng.random((heads, nb, nb)) < c["density"]).astype(np.uint8)
    for h in range(heads):
        np.fill_diagonal(mask[h], 1)
    rep = (rng.random(heads) < 0.5).astype(np.uint8) if stride > 1 else np.zeros(heads, np.uint8)
    md = torch.from_numpy(mask).cuda()
    row_ptr, col_idx, order = cba.build_block_csr(md)
    iv_ptr, ivs = cba.build_block_intervals(md)
    kw = dict(block=block, rep_heads=rep, anchor_stride=stride, n_prefix=n_prefix, grid=grid)
    o = cba.sparse_attn_fwd(qd, kd, vd, row_ptr, col_idx, work_order=order, **kw)
    o_iv = cba.sparse_attn_fwd_intervals(qd, kd, vd, iv_ptr, ivs, work_order=order, **kw)
    energy, lse, od = cba.calib_block_energy(qd, kd, vd, block=block, n_prefix=n_prefix, grid=grid)
    e1, l1, o1 = cba.calib_block_energy_ws(qd, kd, vd, block=block, n_prefix=n_prefix, grid=grid)
    taus = rng.uniform(0.5, 0.99, heads)
    sel, votes = cba.select_blocks_by_energy_heads(energy, taus, 0.5, True, n_prefix // block, return_votes=True)
    torch.cuda.synchronize()
    # skip lists: bit-exact
    rp, ci, wo = oracle.build_csr(mask.reshape(-1, nb))
    np.testing.assert_array_equal(row_ptr.cpu().numpy(), rp)
    np.testing.assert_array_equal(col_idx.cpu().numpy()[:rp[-1]], ci)
    np.testing.assert_array_equal(order.cpu().numpy(), wo)
    ip, first, count, _ = oracle.build_intervals(mask.reshape(-1, nb))
    np.testing.assert_array_equal(iv_ptr.cpu().numpy(), ip)
    packed = (first.astype(np.uint32) | (count.astype(np.uint32) << np.uint32(16))).view(np.int32)
    np.testing.assert_array_equal(ivs.cpu().numpy()[:ip[-1]], packed)
    assert torch.equal(o, o_iv)
    # one-pass energies: O and LSE are the dense pass's bits
    assert torch.equal(o1, od) and torch.equal(l1, lse)
    # selection on the GPU's own energies: bit-exact
    ref_sel, ref_votes = oracle.select_blocks(to_host(energy), taus, 0.5, True, n_prefix // block)
    np.testing.assert_array_equal(sel.cpu().numpy(), ref_sel)
    np.testing.assert_array_equal(votes.cpu().numpy(), ref_votes)
    etol = 1e-4 * block if dtype == "bf16" else 1e-5 * block
    for b in range(batch):
        for h in range(heads):
            ref, _ = oracle.sparse_attention_with_repetition(q[b, h], k[b, h], v[b, h], mask[h], block, n_prefix,
                                                             grid, stride, bool(rep[h]))
            assert_close_out(to_host(o)[b, h], ref, dtype, f"case {seed} sparse b{b} h{h}")
            refd, _ = oracle.dense_attention(q[b, h], k[b, h], v[b, h])
            assert_close_out(to_host(od)[b, h], refd, dtype, f"case {seed} energy-pass O b{b} h{h}")
            ref_e = oracle.block_energy(q[b, h], k[b, h], block)
            assert np.abs(to_host(energy)[b, h] - ref_e).max() <= etol
            assert np.abs(to_host(e1)[b, h] - ref_e).max() <= etol
    # repetition detection where the grid has follower rows
    if stride >= 2 and grid[1] >= 2:
        hs, tc = cba.spatial_rep_similarity(qd, kd, lse, stride, n_prefix=n_prefix, grid=grid)
        torch.cuda.synchronize()
        ctol = 1e-4 if dtype == "bf16" else 1e-5
        for b in range(batch):
            for h in range(heads):
                toks, cos = oracle.repetition_cosines(q[b, h], k[b, h], n_prefix, grid, stride)
                assert np.abs(to_host(tc)[b, h][toks] - cos).max() <= ctol
                assert abs(float(to_host(hs)[b, h]) - cos.mean()) <= ctol
