"""GPU parity of spatial-repetition detection (spatial_rep_similarity,
select_rep_heads) through the C ABI binding, against the fp64 oracle on the same
seeded inputs.

Bars: per-token cosines max |d| <= 1e-4 and head means |d| <= 1e-5 for bf16
inputs (fp32 scores, exponentials and sums; the cosine is a ratio of sums of
positive terms, so its error is a few fp32 roundings of the exponent, far below
the 1e-2 output bar); 1e-5 per token on the fp32 path; repetition flags bit-exact
on the same head scores.  Tokens that are not followers must be left untouched."""
import numpy as np
import pytest
import torch

import calibrated_block_sparse_calib_amd as cba
import oracle
from workloads import AttnConfig, get_config, make_qkv
from tests.gpu_util import log, to_host

pytestmark = pytest.mark.gpu

COS_MAX_BF16, MEAN_MAX_BF16 = 1e-4, 1e-5
COS_MAX_F32 = 1e-5


def _cfg(d, grid, n_prefix, stride, dtype="bf16", heads=3, seed=21):
    return AttnConfig(name="rep", heads=heads, head_dim=d, grid=grid, block=32, dtype=dtype, seed=seed,
                      n_prefix=n_prefix, lt=2.0, ls=5.0, anchor_stride=stride)


CASES = [
    # d, grid (F, H, W), n_prefix, stride
    (128, (2, 17, 20), 0, 4),    # N = 680: 40 (f, x) pairs = 2 chunks, ragged key tail of 40
    (64, (3, 9, 10), 64, 3),     # groups of 3 rows: one of the 3 follower waves idles
    (128, (2, 6, 11), 32, 2),    # stride 2: anchor + one follower wave
    (64, (1, 13, 12), 128, 5),   # stride 5: two follower sub-groups per row group
    (128, (2, 8, 8), 0, 4),      # N = 128: keys an exact multiple of the step
    (128, (3, 7, 5), 7, 4),      # text prefix of 7 tokens (not a multiple of any block)
]


def _draws(cfg, n_draws):
    qs, ks = zip(*[make_qkv(cfg, draw=i, with_v=False)[:2] for i in range(n_draws)])
    return np.stack(qs), np.stack(ks)


def _dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return (t.to(torch.bfloat16) if dtype == "bf16" else t).cuda()


def _gpu_similarity(q, k, cfg):
    """lse from the library's dense pass, then the similarity call."""
    qd, kd = _dev(q, cfg.dtype), _dev(k, cfg.dtype)
    _, lse, _ = cba.calib_block_energy(qd, kd, None, block=cfg.block, n_prefix=0)
    head_sim, token_cos = cba.spatial_rep_similarity(qd, kd, lse, cfg.anchor_stride, n_prefix=cfg.n_prefix,
                                                     grid=cfg.grid)
    torch.cuda.synchronize()
    return to_host(head_sim), to_host(token_cos)


def _check_against_oracle(q, k, cfg, head_sim, token_cos, cos_max, mean_max):
    n_draws, heads = q.shape[:2]
    worst = 0.0
    for dr in range(n_draws):
        for h in range(heads):
            score, full = oracle.repetition_score(q[dr, h], k[dr, h], cfg.n_prefix, cfg.grid, cfg.anchor_stride)
            fol = ~np.isnan(full)
            got = token_cos[dr, h]
            assert np.isnan(got[~fol]).all(), f"draw {dr} head {h}: a non-follower token was written"
            err = np.abs(got[fol].astype(np.float64) - full[fol])
            assert err.max() <= cos_max, f"draw {dr} head {h}: cos max err {err.max():.3e}"
            assert abs(float(head_sim[dr, h]) - score) <= mean_max, \
                f"draw {dr} head {h}: head score {head_sim[dr, h]:.7f} vs {score:.7f}"
            # the head score is the mean of the token values the call wrote
            assert abs(float(head_sim[dr, h]) - got[fol].astype(np.float64).mean()) <= 2e-7
            worst = max(worst, float(err.max()))
    return worst


@pytest.mark.parametrize("d,grid,n_prefix,stride", CASES)
def test_rep_similarity_bf16_small(d, grid, n_prefix, stride):
    cfg = _cfg(d, grid, n_prefix, stride)
    log(f"rep similarity bf16 d={d} grid={grid} prefix={n_prefix} stride={stride}")
    q, k = _draws(cfg, 2)
    head_sim, token_cos = _gpu_similarity(q, k, cfg)
    worst = _check_against_oracle(q, k, cfg, head_sim, token_cos, COS_MAX_BF16, MEAN_MAX_BF16)
    log(f"  ok max cos err {worst:.2e}")


def test_rep_similarity_f32_tiny():
    cfg = get_config("tiny")
    log(f"rep similarity f32 tiny grid={cfg.grid} stride={cfg.anchor_stride}")
    q, k = _draws(cfg, cfg.calib_draws)
    head_sim, token_cos = _gpu_similarity(q, k, cfg)
    worst = _check_against_oracle(q, k, cfg, head_sim, token_cos, COS_MAX_F32, COS_MAX_F32)
    log(f"  ok max cos err {worst:.2e}")


def test_rep_similarity_repeating_heads_are_found():
    """Heads whose follower queries copy their anchors' (plus small noise) score near 1
    and are flagged; the others are not.  GPU flags equal the oracle's flags on the
    oracle's own scores, which lie far from gamma here."""
    cfg = _cfg(128, (2, 12, 16), 0, 4, heads=4)
    q, k = _draws(cfg, 2)
    rng = np.random.default_rng(5)
    f_, h_, w_ = cfg.grid
    for h in (1, 3):
        g = q[:, h].reshape(2, f_, h_, w_, -1)
        anchors = (np.arange(h_) // 4) * 4
        g[:] = g[:, :, anchors] + 0.01 * rng.standard_normal(g.shape)
        q[:, h] = g.reshape(2, f_ * h_ * w_, -1)
    q = np.asarray(torch.from_numpy(q.astype(np.float32)).to(torch.bfloat16).float())  # bf16 values
    head_sim, token_cos = _gpu_similarity(q, k, cfg)
    _check_against_oracle(q, k, cfg, head_sim, token_cos, COS_MAX_BF16, MEAN_MAX_BF16)
    ref_scores = np.array([[oracle.repetition_score(q[dr, h], k[dr, h], 0, cfg.grid, 4)[0]
                            for h in range(cfg.heads)] for dr in range(2)])
    gamma = 0.9
    assert np.all(np.abs(ref_scores - gamma) > 1e-2)
    flags = cba.select_rep_heads(torch.from_numpy(head_sim).cuda(), gamma)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_host(flags).astype(np.uint8), oracle.mark_repetition_heads(ref_scores, gamma))
    np.testing.assert_array_equal(to_host(flags).astype(np.uint8), [0, 1, 0, 1])


@pytest.mark.parametrize("draws,heads", [(1, 1), (3, 40), (4, 1000), (7, 3)])
def test_select_rep_heads_bitexact(draws, heads):
    rng = np.random.default_rng(draws * 1000 + heads)
    scores = rng.random((draws, heads)).astype(np.float32)
    gamma = float(scores[0, 0])
    scores[:, heads // 2] = gamma  # a mean exactly at gamma is not marked
    got = cba.select_rep_heads(torch.from_numpy(scores).cuda(), gamma)
    torch.cuda.synchronize()
    ref = oracle.mark_repetition_heads(scores, gamma)
    np.testing.assert_array_equal(to_host(got).astype(np.uint8), ref)
    assert ref[heads // 2] == 0


def test_rep_similarity_deterministic_and_strided():
    """Repeated calls give identical bits; a strided (non-contiguous heads) layout of
    the same values gives the same bits as the contiguous one."""
    cfg = _cfg(128, (2, 17, 20), 0, 4)
    q, k = _draws(cfg, 1)
    qd, kd = _dev(q, "bf16"), _dev(k, "bf16")
    _, lse, _ = cba.calib_block_energy(qd, kd, None, block=32)
    a = cba.spatial_rep_similarity(qd, kd, lse, 4, grid=cfg.grid)
    b = cba.spatial_rep_similarity(qd, kd, lse, 4, grid=cfg.grid)
    # [batch, seq, heads, d] storage viewed as [batch, heads, seq, d]
    qs = qd.transpose(1, 2).contiguous().transpose(1, 2)
    ks = kd.transpose(1, 2).contiguous().transpose(1, 2)
    c = cba.spatial_rep_similarity(qs, ks, lse, 4, grid=cfg.grid)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1].nan_to_num(), b[1].nan_to_num())
    assert torch.equal(a[0], c[0]) and torch.equal(a[1].nan_to_num(), c[1].nan_to_num())
