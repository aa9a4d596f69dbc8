"""GPU parity of the interval skip list (build_block_intervals,
sparse_attn_fwd_intervals) through the C ABI binding.

Runs are bit-exact against the oracle's build_intervals.  Attention through runs
visits the same blocks in the same order as through the CSR list, so its outputs
must be bit-identical to sparse_attn_fwd's on the same mask; one case per dtype
is also checked against the fp64 oracle."""
import numpy as np
import pytest
import torch

import calibrated_block_sparse_calib_amd as cba
import oracle
from workloads import AttnConfig, get_config, make_qkv, random_block_mask, rep_head_flags
from tests.gpu_util import assert_close_out, log, to_dev, to_host

pytestmark = pytest.mark.gpu


def _packed(first, count):
    return (first.astype(np.uint32) | (count.astype(np.uint32) << np.uint32(16))).view(np.int32)


def _band(rows, nkb, width):
    r = np.arange(rows)[:, None] % nkb
    return (np.abs(r - np.arange(nkb)[None, :]) <= width).astype(np.uint8)


MASKS = [
    ("bernoulli 0.3", lambda rng: (rng.random((40, 591)) < 0.3).astype(np.uint8)),
    ("bernoulli 0.9", lambda rng: (rng.random((33, 130)) < 0.9).astype(np.uint8)),
    ("band", lambda rng: _band(64, 200, 7)),
    ("full 64", lambda rng: np.ones((5, 64), np.uint8)),
    ("full 65", lambda rng: np.ones((5, 65), np.uint8)),
    ("empty", lambda rng: np.zeros((9, 129), np.uint8)),
    ("single column", lambda rng: (rng.random((50, 1)) < 0.5).astype(np.uint8)),
    ("runs across chunks", lambda rng: np.tile(np.r_[np.zeros(60), np.ones(70), np.zeros(3), np.ones(130)]
                                               .astype(np.uint8), (3, 1))),
    ("wide rows", lambda rng: (rng.random((6, 65535)) < rng.uniform(0.001, 0.999, (6, 1))).astype(np.uint8)),
    ("one long run", lambda rng: np.pad(np.ones((2, 65533), np.uint8), ((0, 0), (1, 1)))),
]


@pytest.mark.parametrize("name,make", MASKS, ids=[m[0] for m in MASKS])
@pytest.mark.parametrize("exact", [False, True])
def test_intervals_bitexact(name, make, exact):
    m = make(np.random.default_rng(len(name)))
    iv_ptr, ivs = cba.build_block_intervals(torch.from_numpy(m).cuda(), exact=exact)
    torch.cuda.synchronize()
    rp, first, count, _ = oracle.build_intervals(m)
    np.testing.assert_array_equal(iv_ptr.cpu().numpy(), rp)
    np.testing.assert_array_equal(ivs.cpu().numpy()[:rp[-1]], _packed(first, count))
    if exact:
        assert ivs.numel() == max(int(rp[-1]), 1)


def test_intervals_capacity_guard():
    m = (np.random.default_rng(3).random((20, 100)) < 0.5).astype(np.uint8)
    rp, first, count, _ = oracle.build_intervals(m)
    cap = int(rp[-1]) // 2
    lib = cba.load_library()
    md = torch.from_numpy(m).cuda()
    iv_ptr = torch.empty(21, dtype=torch.int32, device="cuda")
    ivs = torch.full((cap + 8,), -7, dtype=torch.int32, device="cuda")
    import ctypes
    st = lib.build_block_intervals(ctypes.c_void_p(md.data_ptr()), 20, 100, ctypes.c_void_p(iv_ptr.data_ptr()),
                                   ctypes.c_void_p(ivs.data_ptr()), cap,
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0
    got = ivs.cpu().numpy()
    np.testing.assert_array_equal(iv_ptr.cpu().numpy(), rp)  # the total tells the caller
    np.testing.assert_array_equal(got[:cap], _packed(first, count)[:cap])
    assert (got[cap:] == -7).all()  # nothing written at or beyond the capacity


def _small_cfg(d, block, grid, n_prefix, dtype="bf16", heads=3, seed=11):
    return AttnConfig(name="small", heads=heads, head_dim=d, grid=grid, block=block, dtype=dtype, seed=seed,
                      n_prefix=n_prefix, lt=2.0, ls=5.0, density_range=(0.3, 0.6), rep_heads_fixed=(1,),
                      anchor_stride=4)


SMALL = [
    (128, 128, (2, 17, 20), 0),
    (64, 64, (3, 9, 10), 64),
    (128, 32, (2, 6, 11), 32),
    (64, 128, (1, 13, 12), 128),
]


def _both(cfg, q, k, v, mask, rep, dtype, fuse=True, order=None):
    md = torch.from_numpy(mask).cuda()
    row_ptr, col_idx, _ = cba.build_block_csr(md)
    iv_ptr, ivs = cba.build_block_intervals(md)
    qd, kd, vd = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    kw = dict(block=cfg.block, rep_heads=rep, anchor_stride=cfg.anchor_stride, fuse_broadcast=fuse,
              n_prefix=cfg.n_prefix, grid=cfg.grid, work_order=order, return_lse=True)
    # zero-filled outputs: without fuse_broadcast the follower rows stay unwritten
    o_c, l_c = cba.sparse_attn_fwd(qd, kd, vd, row_ptr, col_idx, o=torch.zeros_like(qd), **kw)
    o_i, l_i = cba.sparse_attn_fwd_intervals(qd, kd, vd, iv_ptr, ivs, o=torch.zeros_like(qd), **kw)
    torch.cuda.synchronize()
    return o_c, l_c, o_i, l_i


@pytest.mark.parametrize("d,block,grid,n_prefix", SMALL)
@pytest.mark.parametrize("fuse", [True, False])
def test_sparse_intervals_bitidentical_to_csr(d, block, grid, n_prefix, fuse):
    cfg = _small_cfg(d, block, grid, n_prefix)
    log(f"intervals vs csr d={d} B={block} grid={grid} prefix={n_prefix} fuse={fuse}")
    q, k, v = make_qkv(cfg, draw=0)
    mask = random_block_mask(cfg)
    mask[0, 1] = 0  # a row with no block at all (o = 0, lse = -inf)
    rep = rep_head_flags(cfg)
    o_c, l_c, o_i, l_i = _both(cfg, q, k, v, mask, rep, "bf16", fuse)
    assert torch.equal(o_c, o_i)
    assert torch.equal(l_c.nan_to_num(), l_i.nan_to_num())
    if fuse and d == 128 and block == 128:
        outs = []
        for h in range(cfg.heads):
            o, _ = oracle.sparse_attention_with_repetition(q[h], k[h], v[h], mask[h], block, n_prefix, cfg.grid,
                                                           cfg.anchor_stride, bool(rep[h]))
            outs.append(o)
        assert_close_out(to_host(o_i)[0], np.stack(outs), "bf16", "intervals sparse O")


def test_sparse_intervals_f32_tiny_and_work_order():
    cfg = get_config("tiny")
    q, k, v = make_qkv(cfg, draw=0)
    mask = random_block_mask(cfg)
    rep = rep_head_flags(cfg)
    _, _, order = cba.build_block_csr(torch.from_numpy(mask).cuda())
    o_c, l_c, o_i, l_i = _both(cfg, q, k, v, mask, rep, "f32", order=order)
    assert torch.equal(o_c, o_i) and torch.equal(l_c, l_i)
    outs = [oracle.sparse_attention_with_repetition(q[h], k[h], v[h], mask[h], cfg.block, cfg.n_prefix, cfg.grid,
                                                    cfg.anchor_stride, bool(rep[h]))[0] for h in range(cfg.heads)]
    assert_close_out(to_host(o_i)[0], np.stack(outs), "f32", "tiny intervals sparse O")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["wan14_720p", "mochi"])
def test_sparse_intervals_full_size_bitidentical(name):
    """Full sizes in the benchmark's launch configuration: the Wan-14B Bernoulli
    masks with repetition heads, and Mochi's calibrated (banded) masks of its first
    timestep bucket; the run count of each is logged against the kept blocks."""
    cfg = get_config(name)
    q, k, v = make_qkv(cfg, draw=cfg.calib_draws)
    if cfg.mask_mode == "bernoulli":
        mask, rep = random_block_mask(cfg), rep_head_flags(cfg)
    else:
        draws = [make_qkv(cfg, draw=i, with_v=False) for i in range(cfg.calib_draws)]
        qc = torch.from_numpy(np.stack([x[0] for x in draws])).to(torch.bfloat16).cuda()
        kc = torch.from_numpy(np.stack([x[1] for x in draws])).to(torch.bfloat16).cuda()
        energy, _, _ = cba.calib_block_energy(qc, kc, None, block=cfg.block)
        mask = cba.select_blocks_by_energy(energy, cfg.tau, cfg.rho, True, cfg.n_prefix_blocks).cpu().numpy()
        rep = None
        del qc, kc, energy
    o_c, l_c, o_i, l_i = _both(cfg, q, k, v, mask, rep, "bf16")
    assert torch.equal(o_c, o_i) and torch.equal(l_c, l_i)
    rp, _, _, _ = oracle.build_intervals(mask.reshape(-1, cfg.nb))
    log(f"  {name}: {int(mask.sum())} kept blocks in {int(rp[-1])} runs; outputs bit-identical")


def test_sparse_intervals_without_runs():
    """iv_len = 0: no row has a run, so every output is 0 and every LSE -inf."""
    import ctypes
    cfg = _small_cfg(128, 128, (2, 8, 16), 0, heads=2)
    q, k, v = make_qkv(cfg, draw=0)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    o = torch.full_like(qd, 3.0)
    lse = torch.zeros((1, cfg.heads, cfg.seq_len), dtype=torch.float32, device="cuda")
    iv_ptr = torch.zeros(cfg.heads * cfg.nb + 1, dtype=torch.int32, device="cuda")
    desc = cba.make_desc(qd, cfg.block)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    st = cba.load_library().sparse_attn_fwd_intervals(ctypes.byref(desc), P(qd), P(kd), P(vd), P(iv_ptr), None, 0,
                                                      None, None, 1, 0, P(o), P(lse),
                                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0
    assert torch.count_nonzero(o) == 0
    assert torch.isneginf(lse).all()
