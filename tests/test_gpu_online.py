"""GPU parity of the online-search pieces (block_energy_from_lse,
select_blocks_by_energy_heads) through the C ABI binding, against the fp64 oracle.

Bars: energies |dE| <= 1e-4 * (the query block's total weight), which is
calib_block_energy's 1e-4 * block when the LSE is that of the same inputs (each row
then weighs 1); a cached LSE from other inputs weighs row i by exp(lse_i' - lse_i),
up to e^11 here, so the bar scales with it.  Energies from the LSE of the same
inputs are bit-identical to calib_block_energy's sweep; selection is bit-exact on
the same energies."""
import numpy as np
import pytest
import torch

import calibrated_block_sparse_calib_amd as cba
import oracle
from workloads import AttnConfig, get_config, make_qkv
from tests.gpu_util import check_bf16_outputs, log, to_host

pytestmark = pytest.mark.gpu


def _cfg(d, block, grid, n_prefix, dtype="bf16", heads=3, seed=31):
    return AttnConfig(name="online", heads=heads, head_dim=d, grid=grid, block=block, dtype=dtype, seed=seed,
                      n_prefix=n_prefix, lt=2.0, ls=5.0)


def _dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return (t.to(torch.bfloat16) if dtype == "bf16" else t).cuda()


@pytest.mark.parametrize("d,block,grid,n_prefix,dtype", [
    (128, 128, (2, 17, 20), 0, "bf16"),
    (64, 64, (3, 9, 10), 64, "bf16"),
    (128, 32, (2, 6, 11), 32, "bf16"),
    (64, 32, (4, 8, 8), 0, "f32"),
])
def test_energy_from_cached_lse(d, block, grid, n_prefix, dtype):
    """A search at a later step: the LSE cached by the dense pass on draw 0 is reused
    for the energies of draw 1.  Also: the LSE of the same draw reproduces
    calib_block_energy's energies bit for bit."""
    cfg = _cfg(d, block, grid, n_prefix, dtype)
    log(f"cached-LSE energy d={d} B={block} grid={grid} prefix={n_prefix} {dtype}")
    (q0, k0, _), (q1, k1, _) = make_qkv(cfg, draw=0, with_v=False), make_qkv(cfg, draw=1, with_v=False)
    q0d, k0d, q1d, k1d = (_dev(x[None], dtype) for x in (q0, k0, q1, k1))
    e0, lse0, _ = cba.calib_block_energy(q0d, k0d, None, block=block)
    e0_again = cba.block_energy_from_lse(q0d, k0d, lse0, block=block)
    e1 = cba.block_energy_from_lse(q1d, k1d, lse0, block=block)
    torch.cuda.synchronize()
    assert torch.equal(e0, e0_again)
    lse_host = to_host(lse0)[0]
    got = to_host(e1)[0]
    worst = 0.0
    bar = 1e-4 if dtype == "bf16" else 1e-5
    for h in range(cfg.heads):
        ref = oracle.block_energy_from_lse(q1[h], k1[h], lse_host[h].astype(np.float64), block)
        rel = np.abs(got[h] - ref) / ref.sum(axis=1, keepdims=True)  # per query block's total weight
        worst = max(worst, float(rel.max()))
    assert worst <= bar, f"energy error {worst:.3e} of the block total"
    log(f"  ok max |dE| {worst:.2e} of the query block's total weight")


@pytest.mark.parametrize("draws,heads,nb,prefix", [(1, 4, 37, 0), (3, 40, 65, 2), (2, 256, 9, 1), (1, 2, 4096, 0)])
def test_select_per_head_tau_bitexact(draws, heads, nb, prefix):
    rng = np.random.default_rng(draws * 100 + heads)
    energy = rng.gamma(0.6, 1.0, (draws, heads, nb, nb)).astype(np.float32)
    taus = rng.uniform(0.5, 0.99, heads)
    taus[0] = 1.0  # keeps every block
    taus[-1] = 0.0  # keeps the single highest block of each row
    ed = torch.from_numpy(energy).cuda()
    mask, votes = cba.select_blocks_by_energy_heads(ed, taus, 0.5, True, prefix, return_votes=True)
    same_tau = cba.select_blocks_by_energy_heads(ed, [0.9] * heads, 0.5, True, prefix)
    scalar = cba.select_blocks_by_energy(ed, 0.9, 0.5, True, prefix)
    torch.cuda.synchronize()
    ref_m, ref_v = oracle.select_blocks(energy, taus, 0.5, True, prefix)
    np.testing.assert_array_equal(mask.cpu().numpy(), ref_m)
    np.testing.assert_array_equal(votes.cpu().numpy(), ref_v)
    assert torch.equal(same_tau, scalar)


def test_online_search_sequence_small():
    """A short search/reuse sequence on the GPU, every step checked: step 0 searches
    with a dense pass (O and LSE) and selects on its own energies; step 1 reuses the
    mask for sparse attention; step 2 searches again from the cached LSE of step 0.
    Selections are bit-exact against the oracle on the GPU's energies, and the
    step-2 energies are within the energy bar of the oracle's."""
    cfg = _cfg(128, 64, (2, 8, 16), 0, heads=2)
    taus = [0.9, 0.8]
    # V scaled by 1/4 (exact in bf16): these masks keep few blocks, so outputs follow
    # single keys, and |o| >= 4 would put bf16's own spacing (2^-5) above the bar.
    steps = [(q, k, v * 0.25) for q, k, v in (make_qkv(cfg, draw=i) for i in range(3))]
    dev = lambda x: _dev(x[None], "bf16")
    q, k, v = (dev(x) for x in steps[0])
    e0, lse0, o0 = cba.calib_block_energy(q, k, v, block=cfg.block)
    m0 = cba.select_blocks_by_energy_heads(e0, taus, 0.5, True, 0)
    row_ptr, col_idx, _ = cba.build_block_csr(m0)
    q1, k1, v1 = (dev(x) for x in steps[1])
    o1 = cba.sparse_attn_fwd(q1, k1, v1, row_ptr, col_idx, block=cfg.block)
    q2, k2, _ = (dev(x) for x in steps[2])
    e2 = cba.block_energy_from_lse(q2, k2, lse0, block=cfg.block)
    m2 = cba.select_blocks_by_energy_heads(e2, taus, 0.5, True, 0)
    torch.cuda.synchronize()
    ref_m0, _ = oracle.select_blocks(to_host(e0), taus, 0.5, True, 0)
    np.testing.assert_array_equal(m0.cpu().numpy(), ref_m0)
    ref_m2, _ = oracle.select_blocks(to_host(e2), taus, 0.5, True, 0)
    np.testing.assert_array_equal(m2.cpu().numpy(), ref_m2)
    m0n = m0.cpu().numpy()
    q1h, k1h, v1h = steps[1]
    for h in range(cfg.heads):
        ref, _ = oracle.sparse_attention(q1h[h], k1h[h], v1h[h], m0n[h], cfg.block)
        check_bf16_outputs(to_host(o1)[0, h], ref, f"online sparse h{h}")
        ref_e2 = oracle.block_energy_from_lse(steps[2][0][h], steps[2][1][h], to_host(lse0)[0, h].astype(np.float64),
                                              cfg.block)
        assert (np.abs(to_host(e2)[0, h] - ref_e2) / ref_e2.sum(axis=1, keepdims=True)).max() <= 1e-4
