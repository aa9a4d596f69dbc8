"""GPU parity of the one-pass energy sweep (calib_block_energy_ws) against the fp64
oracle: energies |dE| <= 1e-4 * block (bf16), LSE within 1e-3, repeated calls
bit-identical, and the workspace size enforced.  With V, O and the LSE are
bit-identical to calib_block_energy's dense pass and the energies to the one-pass
result without V; O is also checked against the oracle (bf16 max 1e-2 beyond the
output's bf16 rounding, mean 1e-3)."""
import ctypes

import numpy as np
import pytest
import torch

import calibrated_block_sparse_calib_amd as cba
import oracle
from workloads import AttnConfig, get_config, make_qkv
from tests.gpu_util import assert_close_lse, assert_close_out, log, to_host

pytestmark = pytest.mark.gpu


def _cfg(d, block, grid, n_prefix, heads=3):
    return AttnConfig(name="e1", heads=heads, head_dim=d, grid=grid, block=block, dtype="bf16", seed=41,
                      n_prefix=n_prefix, lt=2.0, ls=5.0)


@pytest.mark.parametrize("d,block,grid,n_prefix", [
    (128, 128, (2, 17, 20), 0),   # ragged last block of 40
    (64, 64, (3, 9, 10), 64),
    (128, 32, (2, 6, 11), 32),
    (64, 128, (1, 13, 12), 128),
    (128, 64, (2, 8, 8), 0),      # exact multiple
    (128, 128, (1, 1, 5), 0),     # one short block
    (64, 32, (2, 5, 7), 32),      # ragged last block of 6, text prefix
])
def test_onepass_energy_matches_oracle(d, block, grid, n_prefix):
    cfg = _cfg(d, block, grid, n_prefix)
    log(f"one-pass energy d={d} B={block} grid={grid} prefix={n_prefix}")
    draws = [make_qkv(cfg, draw=i) for i in range(2)]
    q = np.stack([x[0] for x in draws])
    k = np.stack([x[1] for x in draws])
    v = np.stack([x[2] for x in draws])
    qd, kd, vd = (torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda() for x in (q, k, v))
    e1, l1, _ = cba.calib_block_energy_ws(qd, kd, block=block)
    e1b, l1b, _ = cba.calib_block_energy_ws(qd, kd, block=block)
    e2, l2, _ = cba.calib_block_energy(qd, kd, None, block=block)
    ev, lv, ov = cba.calib_block_energy_ws(qd, kd, vd, block=block)
    _, l2v, o2v = cba.calib_block_energy(qd, kd, vd, block=block)
    torch.cuda.synchronize()
    assert torch.equal(e1, e1b) and torch.equal(l1, l1b)
    assert torch.equal(ov, o2v) and torch.equal(lv, l2v) and torch.equal(lv, l1)
    assert torch.equal(ev, e1)
    for dr in range(2):
        refd, _ = oracle.dense_attention(q[dr, 0], k[dr, 0], v[dr, 0])
        assert_close_out(to_host(ov)[dr, 0], refd, "bf16", f"one-pass O draw {dr}")
    got_e, got_l = to_host(e1), to_host(l1)
    worst = 0.0
    for dr in range(2):
        for h in range(cfg.heads):
            ref = oracle.block_energy(q[dr, h], k[dr, h], block)
            worst = max(worst, float(np.abs(got_e[dr, h] - ref).max()))
            _, ref_lse = oracle.dense_attention(q[dr, h], k[dr, h], k[dr, h])
            assert_close_lse(got_l[dr, h], ref_lse, f"one-pass LSE draw {dr} head {h}", 1e-3)
    assert worst <= 1e-4 * block, f"energy error {worst:.3e}"
    # against the two-sweep energies of the same inputs
    assert float((e1 - e2).abs().max()) <= 2e-4 * block
    log(f"  ok max |dE| {worst:.2e}")


@pytest.mark.parametrize("block,fraction", [(128, 0.999), (128, 0.3), (64, 0.25), (32, 0.2)])
def test_onepass_partial_workspace_runs_in_chunks(block, fraction):
    """A workspace smaller than the whole problem's runs the pass in several launches:
    energies, LSE and O bit-identical to the single launch with a full workspace."""
    cfg = _cfg(128, block, (2, 8, 16), 0)
    draws = [make_qkv(cfg, draw=i) for i in range(2)]
    dev = lambda i: torch.from_numpy(np.ascontiguousarray(np.stack([x[i] for x in draws]))).to(torch.bfloat16).cuda()
    qd, kd, vd = dev(0), dev(1), dev(2)
    need = cba.energy_workspace_bytes(qd, block)
    for v in (None, vd):
        e_full, l_full, o_full = cba.calib_block_energy_ws(qd, kd, v, block=block)
        ws = torch.empty(int(need * fraction) // 16 * 16, dtype=torch.uint8, device="cuda")
        e, l, o = cba.calib_block_energy_ws(qd, kd, v, block=block, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(e, e_full) and torch.equal(l, l_full)
        if v is not None:
            assert torch.equal(o, o_full)
    log(f"  ok block {block}: workspace {fraction:.3f} of {need} bytes, bit-identical")


def test_onepass_workspace_too_small_is_refused():
    cfg = _cfg(128, 128, (2, 8, 16), 0)
    q, k, _ = make_qkv(cfg, draw=0, with_v=False)
    qd = torch.from_numpy(q[None]).to(torch.bfloat16).cuda()
    kd = torch.from_numpy(k[None]).to(torch.bfloat16).cuda()
    nb = cba.n_blocks(qd.shape[2], 128)
    one_group = 2 * nb * 128 * 4  # two query blocks per workgroup without V
    ws = torch.empty(one_group - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(cba.CalibAttnError):
        cba.calib_block_energy_ws(qd, kd, block=128, workspace=ws)


@pytest.mark.timeout(600)
def test_onepass_energy_full_size_hunyuan():
    """HunyuanVideo shape, one draw: sampled query blocks against the oracle and the
    whole energy tensor against the two-sweep result."""
    cfg = get_config("hunyuan")
    q, k, _ = make_qkv(cfg, draw=0, with_v=False)
    qd = torch.from_numpy(q[None]).to(torch.bfloat16).cuda()
    kd = torch.from_numpy(k[None]).to(torch.bfloat16).cuda()
    e1, l1, _ = cba.calib_block_energy_ws(qd, kd, block=cfg.block)
    e2, l2, _ = cba.calib_block_energy(qd, kd, None, block=cfg.block)
    torch.cuda.synchronize()
    assert float((e1 - e2).abs().max()) <= 2e-4 * cfg.block
    assert float((l1 - l2).abs().max()) <= 1e-3
    got = to_host(e1)[0]
    rng = np.random.default_rng(4)
    worst = 0.0
    for h, qb in [(0, 0), (cfg.heads - 1, cfg.nb - 1)] + [(int(a), int(b)) for a, b in
                                                          zip(rng.integers(0, cfg.heads, 4), rng.integers(0, cfg.nb, 4))]:
        ref = oracle.block_energy(q[h], k[h], cfg.block, q_blocks=[qb])[0]
        worst = max(worst, float(np.abs(got[h, qb] - ref).max()))
    log(f"  hunyuan one-pass: max |dE| {worst:.2e} on sampled rows")
    assert worst <= 1e-4 * cfg.block
