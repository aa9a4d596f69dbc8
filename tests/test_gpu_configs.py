"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (natural row order, fused broadcast).  The fp64 oracle cannot
run these sizes in full, so each test samples query blocks of every head --
always the first, the ragged last one and the text blocks, plus seeded random
ones -- and checks:

  * block energies of the sampled rows: |dE| <= 1e-4 * block;
  * selection on the GPU's own energies: bit-exact vs the oracle's selection;
  * the calibrated mask vs the oracle's calibration from its own fp64 energies:
    >= 99.9% of the sampled blocks agree, and every differing block lies in a
    row where, in some draw, a cumulative energy fraction of the oracle's
    order is within 1e-4 of tau (its keep decision flips when tau moves by
    1e-4).  The number of differing blocks is printed;
  * the skip list of the whole mask: bit-exact;
  * attention outputs of the sampled rows: bf16 bars (max 1e-2 beyond the
    output's bf16 rounding, mean 1e-3).
"""
import numpy as np
import pytest
import torch

import calibrated_block_sparse_calib_amd as cba
import oracle
from workloads import get_config, make_qkv, random_block_mask, rep_head_flags
from tests.gpu_util import assert_close_out, check_bf16_outputs, log

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

TIE_TAU = 1e-4  # the tau tie window


def _sample_blocks(cfg, per_head, seed):
    """(head, query block) pairs: for every head the first, the ragged last and the
    text blocks plus per_head seeded random ones."""
    rng = np.random.default_rng(seed)
    fixed = sorted({0, cfg.nb - 1} | set(range(cfg.n_prefix_blocks)))
    picks = set()
    for h in range(cfg.heads):
        picks |= {(h, qb) for qb in fixed}
        picks |= {(h, int(qb)) for qb in rng.integers(0, cfg.nb, per_head)}
    return sorted(picks)


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda()


def _tau_ties(e_draws, tau):
    """Blocks whose keep decision flips in at least one draw when tau moves by 1e-4:
    a cumulative energy fraction of the oracle's order lies within 1e-4 of tau."""
    amb = np.zeros(e_draws.shape[1], dtype=bool)
    for e in e_draws:
        lo = oracle.select_row(e, tau - TIE_TAU)
        hi = oracle.select_row(e, min(tau + TIE_TAU, 1.0))
        amb |= lo != hi
    return amb


def _calibrate_and_check(cfg, bucket=0, per_head=2, seed=0):
    """GPU calibration of one workload (bucket) + sampled oracle checks.
    Returns (mask, eval inputs) for the attention check."""
    log(f"calibrating {cfg.name} bucket {bucket}")
    draws = [make_qkv(cfg, draw=d, bucket=bucket, with_v=False) for d in range(cfg.calib_draws)]
    q = np.stack([d[0] for d in draws])
    k = np.stack([d[1] for d in draws])
    energy, _, _ = cba.calib_block_energy(_dev(q), _dev(k), None, block=cfg.block)
    mask, votes = cba.select_blocks_by_energy(energy, cfg.tau, cfg.rho, True, cfg.n_prefix_blocks, return_votes=True)
    torch.cuda.synchronize()
    e_gpu = energy.cpu().numpy()
    m_gpu = mask.cpu().numpy()
    picks = _sample_blocks(cfg, per_head, seed)
    B = cfg.block
    agree, total, worst_e, n_tau = 0, 0, 0.0, 0
    votes_np = votes.cpu().numpy()
    for h, qb in picks:
        e_ref = np.stack([oracle.block_energy(q[d, h], k[d, h], B, q_blocks=[qb])[0] for d in range(cfg.calib_draws)])
        worst_e = max(worst_e, float(np.abs(e_gpu[:, h, qb] - e_ref).max()))
        # selection on the GPU's own energies: bit-exact
        m_same, v_same = oracle.select_blocks(e_gpu[:, h:h + 1, qb:qb + 1], cfg.tau, cfg.rho, False, 0)
        forced = np.zeros(cfg.nb, dtype=bool)
        forced[qb] = True
        if qb < cfg.n_prefix_blocks:
            forced[:] = True
        forced[:cfg.n_prefix_blocks] = True
        np.testing.assert_array_equal(votes_np[h, qb], v_same[0, 0])
        np.testing.assert_array_equal(m_gpu[h, qb].astype(bool), m_same[0, 0].astype(bool) | forced)
        # calibrated mask vs the oracle's own calibration
        m_ref, _ = oracle.select_blocks(e_ref[:, None, None, :], cfg.tau, cfg.rho, False, 0)
        m_ref = m_ref[0, 0].astype(bool) | forced
        diff = m_gpu[h, qb].astype(bool) != m_ref
        if diff.any():
            tau_tie = _tau_ties(e_ref, cfg.tau)
            other = diff & ~tau_tie
            assert not other.any(), f"{cfg.name} h{h} qb{qb}: mask differences at {np.nonzero(other)[0]} are not ties"
            n_tau += int(diff.sum())
        agree += int((~diff).sum())
        total += diff.size
    assert worst_e <= 1e-4 * B, f"energy error {worst_e:.3e}"
    assert agree / total >= 0.999, f"mask agreement {agree / total:.5f}"
    log(f"  {cfg.name} b{bucket}: {len(picks)} sampled rows, energy max err {worst_e:.2e}, mask agreement "
        f"{agree}/{total}, differing blocks (all at tau ties): {n_tau}; "
        f"density {m_gpu.mean():.3f}")
    # skip list of the whole mask: bit-exact
    row_ptr, col_idx, order = cba.build_block_csr(mask)
    torch.cuda.synchronize()
    rp_ref, ci_ref, wo_ref = oracle.build_csr(m_gpu.reshape(-1, cfg.nb))
    np.testing.assert_array_equal(row_ptr.cpu().numpy(), rp_ref)
    np.testing.assert_array_equal(col_idx.cpu().numpy()[:rp_ref[-1]], ci_ref)
    np.testing.assert_array_equal(order.cpu().numpy(), wo_ref)
    del energy
    return m_gpu, mask, row_ptr, col_idx


def _check_attention(cfg, q, k, v, m_np, row_ptr, col_idx, rep, per_head, seed, bucket=0):
    qd, kd, vd = _dev(q[None]), _dev(k[None]), _dev(v[None])
    o = cba.sparse_attn_fwd(qd, kd, vd, row_ptr, col_idx, block=cfg.block, rep_heads=rep,
                            anchor_stride=cfg.anchor_stride, fuse_broadcast=True, n_prefix=cfg.n_prefix,
                            grid=cfg.grid)
    torch.cuda.synchronize()
    got = o[0].float().cpu().numpy()
    gots, refs = [], []
    for h, qb in _sample_blocks(cfg, per_head, seed + 1):
        lo, hi = qb * cfg.block, min(cfg.seq_len, (qb + 1) * cfg.block)
        is_rep = bool(rep is not None and rep[h])
        rows = np.zeros(cfg.seq_len, dtype=bool)
        rows[lo:hi] = oracle.computed_rows(cfg.seq_len, cfg.n_prefix, cfg.grid, cfg.anchor_stride, is_rep)[lo:hi]
        ref, _ = oracle.sparse_attention(q[h], k[h], v[h], m_np[h], cfg.block, None, rows)
        gots.append(got[h][rows])
        refs.append(ref[rows])
        if is_rep:
            # followers carry their anchor's output exactly
            full = oracle.row_broadcast(got[h], cfg.n_prefix, cfg.grid, cfg.anchor_stride)
            np.testing.assert_array_equal(full[lo:hi], got[h][lo:hi])
    g_all, r_all = np.concatenate(gots), np.concatenate(refs)
    mx, mx_exc, mean = check_bf16_outputs(g_all, r_all, f"{cfg.name} b{bucket} sparse")
    log(f"  {cfg.name} b{bucket} sparse: rows {g_all.shape[0]} max {mx:.3e} (beyond bf16 rounding {mx_exc:.3e}) "
        f"mean {mean:.3e}")
    return qd, kd, vd


def test_wan13_480p_calibration_and_sparse():
    cfg = get_config("wan13_480p")
    m_np, mask, row_ptr, col_idx = _calibrate_and_check(cfg, per_head=6, seed=1)
    q, k, v = make_qkv(cfg, draw=cfg.calib_draws)
    _check_attention(cfg, q, k, v, m_np, row_ptr, col_idx, None, 6, 1)
    assert 0.2 <= m_np.mean() <= 0.4


def test_mochi_buckets():
    cfg = get_config("mochi")
    for bucket in range(cfg.buckets):
        m_np, mask, row_ptr, col_idx = _calibrate_and_check(cfg, bucket=bucket, per_head=3, seed=10 + bucket)
        assert m_np[:, :2, :].all() and m_np[:, :, :2].all()  # text rows and columns dense
        q, k, v = make_qkv(cfg, draw=cfg.calib_draws, bucket=bucket)
        _check_attention(cfg, q, k, v, m_np, row_ptr, col_idx, None, 4, 20 + bucket, bucket)


def test_hunyuan_calibration_and_sparse():
    cfg = get_config("hunyuan")
    m_np, mask, row_ptr, col_idx = _calibrate_and_check(cfg, per_head=2, seed=3)
    dens = m_np.mean(axis=(1, 2))
    log(f"  hunyuan per-head density {np.round(dens, 2).tolist()}")
    assert dens.min() < 0.2 and dens.max() > 0.5  # head-adaptive spread
    q, k, v = make_qkv(cfg, draw=cfg.calib_draws)
    _check_attention(cfg, q, k, v, m_np, row_ptr, col_idx, None, 4, 3)


def test_wan14_720p_sparse_dense_and_repetition():
    """The benchmark's workload: seeded masks, 10 repetition heads, fused broadcast;
    then the unfused broadcast path, the longest-first order and dense attention."""
    cfg = get_config("wan14_720p")
    q, k, v = make_qkv(cfg, draw=cfg.calib_draws)
    m_np = random_block_mask(cfg)
    rep = rep_head_flags(cfg)
    mask = torch.from_numpy(m_np).cuda()
    row_ptr, col_idx, order = cba.build_block_csr(mask)
    torch.cuda.synchronize()
    rp_ref, ci_ref, wo_ref = oracle.build_csr(m_np.reshape(-1, cfg.nb))
    np.testing.assert_array_equal(row_ptr.cpu().numpy(), rp_ref)
    np.testing.assert_array_equal(order.cpu().numpy(), wo_ref)
    qd, kd, vd = _check_attention(cfg, q, k, v, m_np, row_ptr, col_idx, rep, 4, 5)
    # same kernel through the explicit order and the separate broadcast: identical bits
    o_fused = cba.sparse_attn_fwd(qd, kd, vd, row_ptr, col_idx, block=cfg.block, rep_heads=rep,
                                  anchor_stride=cfg.anchor_stride, fuse_broadcast=True, grid=cfg.grid)
    o_split = cba.sparse_attn_fwd(qd, kd, vd, row_ptr, col_idx, block=cfg.block, work_order=order, rep_heads=rep,
                                  anchor_stride=cfg.anchor_stride, fuse_broadcast=False, grid=cfg.grid)
    cba.rep_row_broadcast(o_split, rep, cfg.anchor_stride, block=cfg.block, grid=cfg.grid)
    torch.cuda.synchronize()
    assert torch.equal(o_fused, o_split)
    del o_fused, o_split
    # dense attention on sampled rows
    od = cba.dense_attn_fwd(qd, kd, vd, block=cfg.block)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    heads = rng.integers(0, cfg.heads, 4)
    gots, refs = [], []
    for h in heads:
        rows = np.sort(rng.choice(cfg.seq_len, 48, replace=False))
        rows[-1] = cfg.seq_len - 1
        want = np.zeros(cfg.seq_len, dtype=bool)
        want[rows] = True
        ref, _ = oracle.sparse_attention(q[h], k[h], v[h], np.ones((cfg.nb, cfg.nb), bool), cfg.block, None, want)
        gots.append(od[0, h].float().cpu().numpy()[rows])
        refs.append(ref[rows])
    mx, mx_exc, mean = check_bf16_outputs(np.concatenate(gots), np.concatenate(refs), "wan14_720p dense")
    log(f"  wan14_720p dense: rows {len(heads) * 48} max {mx:.3e} (beyond bf16 rounding {mx_exc:.3e}) "
        f"mean {mean:.3e}")


@pytest.mark.parametrize("name", ["wan14_720p", "mochi"])
def test_repetition_detection_full_size(name):
    """spatial_rep_similarity on one full-size draw (the launch the benchmark times):
    sampled follower tokens of a few heads against the oracle (max 1e-4), every head
    score equal to the mean of the token values written, and the flags of
    select_rep_heads bit-exact against the oracle's rule on the GPU's scores."""
    cfg = get_config(name)
    q, k, _ = make_qkv(cfg, draw=0, with_v=False)
    qd, kd = _dev(q[None]), _dev(k[None])
    _, lse, _ = cba.calib_block_energy(qd, kd, None, block=cfg.block, n_prefix=cfg.n_prefix, grid=cfg.grid)
    head_sim, token_cos = cba.spatial_rep_similarity(qd, kd, lse, cfg.anchor_stride, n_prefix=cfg.n_prefix,
                                                     grid=cfg.grid)
    torch.cuda.synchronize()
    hs = head_sim.cpu().numpy()
    tc = token_cos[0].cpu().numpy()
    f_, h_, w_ = cfg.grid
    t = np.arange(cfg.n_prefix, cfg.seq_len)
    fol_mask = np.zeros(cfg.seq_len, dtype=bool)
    fol_mask[t[((t - cfg.n_prefix) // w_) % h_ % cfg.anchor_stride != 0]] = True
    assert np.isnan(tc[:, ~fol_mask]).all() and np.isfinite(tc[:, fol_mask]).all()
    np.testing.assert_allclose(hs[0], tc[:, fol_mask].astype(np.float64).mean(axis=1), atol=2e-7, rtol=0)
    rng = np.random.default_rng(9)
    fol = np.nonzero(fol_mask)[0]
    errs = []
    for h in sorted({0, cfg.heads - 1, int(rng.integers(0, cfg.heads))}):
        pick = np.unique(np.concatenate([rng.choice(fol, 64, replace=False), fol[:2], fol[-2:]]))
        _, ref = oracle.repetition_cosines(q[h], k[h], cfg.n_prefix, cfg.grid, cfg.anchor_stride, tokens=pick)
        errs.append(np.abs(tc[h][pick].astype(np.float64) - ref))
    err = np.concatenate(errs)
    log(f"  {name} repetition: {err.size} tokens, max err {err.max():.2e}; head scores "
        f"{hs.min():.3f}..{hs.max():.3f}")
    assert err.max() <= 1e-4
    gamma = float(np.median(hs))
    flags = cba.select_rep_heads(head_sim, gamma)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(flags.cpu().numpy(), oracle.mark_repetition_heads(hs, gamma))
