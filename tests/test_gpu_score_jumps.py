"""Large score jumps after a row's first key block: the online softmax must raise
its running reference (with the lazy rescale) however far the scores climb.  The
inputs put mild jumps (up to 65 base-2 units), jumps far beyond the fp32 range of
exp2 against the first block's maximum (147 units), and work items where only
some rows jump.  Every output must be finite and within the usual bf16 bars of
the fp64 oracle, and the CSR and interval paths must agree bit for bit."""
import numpy as np
import pytest
import torch

import calibrated_block_sparse_calib_amd as cba
import oracle
from tests.gpu_util import assert_close_lse, assert_close_out, log, to_host

pytestmark = pytest.mark.gpu

D = 128
# c * |u|^2 = 128 / sqrt(128) * log2(e) = 16.3 base-2 units of score per unit of alpha.
CASES = {
    "none": (0, 0, 0, 0, 0),       # no jump
    "mild": (0, 1, 2, 3, 4),       # up to 65 units above the first block
    "overflow": (0, 0, 9, 0, 9),   # 147 units: exp2 against the first block's maximum would overflow
}


def _inputs(alpha, block, n, heads, mixed, seed):
    rng = np.random.default_rng(seed)
    u = np.where(rng.random(D) < 0.5, -1.0, 1.0)
    q = 0.3 * rng.standard_normal((heads, n, D))
    k = 0.3 * rng.standard_normal((heads, n, D))
    v = rng.standard_normal((heads, n, D))
    sign = np.ones(n)
    if mixed:  # half the rows of every block look away from the jump
        sign[(np.arange(n) // 16) % 2 == 1] = -1.0
    q += sign[None, :, None] * u[None, None, :]
    kb = np.arange(n) // 128  # alpha per 128 tokens, whatever the block size
    k += np.asarray(alpha, np.float64)[np.minimum(kb, len(alpha) - 1)][None, :, None] * u[None, None, :]
    to_bf = lambda a: torch.from_numpy(a.astype(np.float32)[None]).to(torch.bfloat16)
    qt, kt, vt = to_bf(q), to_bf(k), to_bf(v)
    return (qt.float().numpy()[0], kt.float().numpy()[0], vt.float().numpy()[0]), (qt.cuda(), kt.cuda(), vt.cuda())


@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("block", [128, 64])
@pytest.mark.parametrize("mixed", [False, True])
def test_large_score_jumps(case, block, mixed):
    heads, n = 2, 600  # 5 blocks of 128 tokens, the last ragged
    log(f"score jumps case={case} B={block} mixed={mixed}")
    (q, k, v), (qd, kd, vd) = _inputs(CASES[case], block, n, heads, mixed, seed=block + 7 * mixed)
    nb = (n + block - 1) // block
    rng = np.random.default_rng(nb)
    mask = (rng.random((heads, nb, nb)) < 0.5).astype(np.uint8)
    mask[:, :, 0] = 1  # every row starts at key block 0, which holds no jump
    mask[:, :, nb - 1] = 1
    row_ptr, col_idx, order = cba.build_block_csr(torch.from_numpy(mask).cuda())
    iv_ptr, ivs = cba.build_block_intervals(torch.from_numpy(mask).cuda())
    o = cba.sparse_attn_fwd(qd, kd, vd, row_ptr, col_idx, block=block, work_order=order)
    o2, lse = cba.sparse_attn_fwd(qd, kd, vd, row_ptr, col_idx, block=block, return_lse=True)
    oi = cba.sparse_attn_fwd_intervals(qd, kd, vd, iv_ptr, ivs, block=block)
    od, lsed = cba.dense_attn_fwd(qd, kd, vd, block=block, return_lse=True)
    torch.cuda.synchronize()
    for name, t in (("sparse", o), ("sparse with LSE", o2), ("intervals", oi), ("dense", od)):
        assert torch.isfinite(t).all(), f"{name}: non-finite values"
    assert torch.equal(o, oi) and torch.equal(o, o2)
    for h in range(heads):
        ref, ref_lse = oracle.sparse_attention(q[h], k[h], v[h], mask[h], block)
        assert_close_out(to_host(o)[0, h], ref, "bf16", f"{case} sparse h{h}")
        assert_close_lse(to_host(lse)[0, h], ref_lse, f"{case} sparse h{h}", 1e-3)
        refd, refd_lse = oracle.dense_attention(q[h], k[h], v[h])
        assert_close_out(to_host(od)[0, h], refd, "bf16", f"{case} dense h{h}")
        assert_close_lse(to_host(lsed)[0, h], refd_lse, f"{case} dense h{h}", 1e-3)
