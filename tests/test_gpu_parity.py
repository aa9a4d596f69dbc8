"""GPU parity: every entry point of libcalibattn.so, called through the C ABI
binding, against the fp64 oracle on the same seeded inputs.

Small cases run the oracle in full: the tiny fp32 workload and bf16 grids that
span several query and key blocks with a ragged last block, text tokens and a
repetition head.  Bars: masks, CSR, work order and broadcast copies bit-exact;
bf16 outputs max |d| <= 1e-2 beyond
the output's bf16 rounding and mean |d| <= 1e-3; fp32 outputs max |d| <= 1e-5."""
import numpy as np
import pytest
import torch

import calibrated_block_sparse_calib_amd as cba
import oracle
from workloads import AttnConfig, get_config, make_qkv, random_block_mask, rep_head_flags
from tests.gpu_util import assert_close_lse, assert_close_out, log, to_dev, to_host

pytestmark = pytest.mark.gpu


def _small_cfg(d, block, grid, n_prefix, dtype="bf16", heads=3, seed=11):
    return AttnConfig(name="small", heads=heads, head_dim=d, grid=grid, block=block, dtype=dtype, seed=seed,
                      n_prefix=n_prefix, lt=2.0, ls=5.0, density_range=(0.3, 0.6), rep_heads_fixed=(1,),
                      anchor_stride=4)


SMALL = [
    (128, 128, (2, 17, 20), 0),    # N = 680: 6 blocks, last holds 40
    (64, 64, (3, 9, 10), 64),      # N = 334: text block + ragged tail of 14
    (128, 32, (2, 6, 11), 32),     # N = 164: 6 blocks, last holds 4
    (64, 128, (1, 13, 12), 128),   # N = 284: last holds 28
    (128, 64, (2, 8, 8), 0),       # N = 128: exact multiple of the block
]


def _oracle_sparse(cfg, q, k, v, mask, rep, stride):
    outs, lses = [], []
    for h in range(cfg.heads):
        o, l = oracle.sparse_attention_with_repetition(q[h], k[h], v[h], mask[h], cfg.block, cfg.n_prefix,
                                                       cfg.grid, stride, bool(rep[h]))
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


@pytest.mark.parametrize("d,block,grid,n_prefix", SMALL)
@pytest.mark.parametrize("fuse,use_order", [(True, True), (False, True), (True, False)])
def test_sparse_bf16_small(d, block, grid, n_prefix, fuse, use_order):
    """use_order=False processes the rows in natural order."""
    cfg = _small_cfg(d, block, grid, n_prefix)
    log(f"sparse bf16 d={d} B={block} grid={grid} prefix={n_prefix} fuse={fuse} order={use_order}")
    q, k, v = make_qkv(cfg, draw=0)
    mask = random_block_mask(cfg)
    if cfg.nb > 2:
        mask[2, 1, :] = 0  # a query block that keeps nothing
    rep = rep_head_flags(cfg)
    dm = torch.from_numpy(mask).cuda()
    row_ptr, col_idx, order = cba.build_block_csr(dm)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    o, lse = cba.sparse_attn_fwd(qd, kd, vd, row_ptr, col_idx, block=block,
                                 work_order=order if use_order else None, rep_heads=rep,
                                 anchor_stride=4, fuse_broadcast=fuse, n_prefix=n_prefix, grid=grid,
                                 return_lse=True)
    if not fuse:
        cba.rep_row_broadcast(o, rep, 4, block=block, n_prefix=n_prefix, grid=grid)
    torch.cuda.synchronize()
    ref_o, ref_l = _oracle_sparse(cfg, q, k, v, mask, rep, 4)
    assert_close_out(to_host(o)[0], ref_o, "bf16", "sparse O")
    assert_close_lse(to_host(lse)[0], ref_l, "sparse", 1e-3)


@pytest.mark.parametrize("d,block,grid,n_prefix", SMALL[:3])
def test_dense_bf16_small(d, block, grid, n_prefix):
    cfg = _small_cfg(d, block, grid, n_prefix)
    q, k, v = make_qkv(cfg, draw=1)
    o, lse = cba.dense_attn_fwd(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), block=block,
                                return_lse=True)
    torch.cuda.synchronize()
    for h in range(cfg.heads):
        ro, rl = oracle.dense_attention(q[h], k[h], v[h])
        assert_close_out(to_host(o)[0, h], ro, "bf16", f"dense O head {h}")
        assert_close_lse(to_host(lse)[0, h], rl, "dense", 1e-3)


@pytest.mark.parametrize("d,block,grid,n_prefix", SMALL[:4])
def test_energy_bf16_small(d, block, grid, n_prefix):
    cfg = _small_cfg(d, block, grid, n_prefix)
    draws = [make_qkv(cfg, draw=i) for i in range(2)]
    q = np.stack([x[0] for x in draws])
    k = np.stack([x[1] for x in draws])
    v = np.stack([x[2] for x in draws])
    qd = torch.from_numpy(q).to(torch.bfloat16).cuda()
    kd = torch.from_numpy(k).to(torch.bfloat16).cuda()
    vd = torch.from_numpy(v).to(torch.bfloat16).cuda()
    energy, lse, o = cba.calib_block_energy(qd, kd, vd, block=block)
    torch.cuda.synchronize()
    e = to_host(energy)
    for dr in range(2):
        for h in range(cfg.heads):
            ref = oracle.block_energy(q[dr, h], k[dr, h], block)
            err = np.abs(e[dr, h] - ref).max()
            assert err <= 1e-4 * block, f"energy draw {dr} head {h}: {err:.3e}"
            ro, rl = oracle.dense_attention(q[dr, h], k[dr, h], v[dr, h])
            assert_close_out(to_host(o)[dr, h], ro, "bf16", "energy sweep-1 O")
            assert_close_lse(to_host(lse)[dr, h], rl, "energy sweep-1", 1e-3)
    # without V: LSE only, same energies bit for bit
    e2, lse2, o2 = cba.calib_block_energy(qd, kd, None, block=block)
    torch.cuda.synchronize()
    assert o2 is None
    np.testing.assert_array_equal(to_host(e2), e)


# ---------------------------------------------------------------- tiny fp32 workload

@pytest.fixture(scope="module")
def tiny():
    cfg = get_config("tiny")
    calib = [make_qkv(cfg, draw=i) for i in range(cfg.calib_draws)]
    evalq = make_qkv(cfg, draw=cfg.calib_draws)
    return cfg, calib, evalq


def test_tiny_dense_f32(tiny):
    cfg, _, (q, k, v) = tiny
    o, lse = cba.dense_attn_fwd(to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32"), block=cfg.block,
                                return_lse=True)
    torch.cuda.synchronize()
    for h in range(cfg.heads):
        ro, rl = oracle.dense_attention(q[h], k[h], v[h])
        assert_close_out(to_host(o)[0, h], ro, "f32", "tiny dense")
        assert_close_lse(to_host(lse)[0, h], rl, "tiny dense", 1e-5)


def test_tiny_calibration_f32(tiny):
    """Full calibration on the tiny workload: energies, GPU selection vs the oracle's
    selection on the same energies (bit-exact), then vs the oracle's own energies."""
    cfg, calib, _ = tiny
    q = np.stack([c[0] for c in calib])
    k = np.stack([c[1] for c in calib])
    energy, lse, _ = cba.calib_block_energy(torch.from_numpy(q).cuda(), torch.from_numpy(k).cuda(), None,
                                            block=cfg.block)
    mask, votes = cba.select_blocks_by_energy(energy, cfg.tau, cfg.rho, True, 0, return_votes=True)
    torch.cuda.synchronize()
    e = to_host(energy)
    ref_e = np.stack([np.stack([oracle.block_energy(q[d, h], k[d, h], cfg.block) for h in range(cfg.heads)])
                      for d in range(cfg.calib_draws)])
    assert np.abs(e - ref_e).max() <= 1e-5 * cfg.block
    m_same, v_same = oracle.select_blocks(e, cfg.tau, cfg.rho, True, 0)
    np.testing.assert_array_equal(mask.cpu().numpy(), m_same)
    np.testing.assert_array_equal(votes.cpu().numpy(), v_same)
    m_ref, _ = oracle.select_blocks(ref_e, cfg.tau, cfg.rho, True, 0)
    agree = (mask.cpu().numpy() == m_ref).mean()
    assert agree >= 0.999, agree


def test_tiny_sparse_f32_with_repetition(tiny):
    cfg, _, (q, k, v) = tiny
    mask = random_block_mask(cfg)
    rep = rep_head_flags(cfg)
    row_ptr, col_idx, order = cba.build_block_csr(torch.from_numpy(mask).cuda())
    for fuse in (True, False):
        o, lse = cba.sparse_attn_fwd(to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32"), row_ptr, col_idx,
                                     block=cfg.block, work_order=order, rep_heads=rep, anchor_stride=cfg.anchor_stride,
                                     fuse_broadcast=fuse, grid=cfg.grid, return_lse=True)
        if not fuse:
            cba.rep_row_broadcast(o, rep, cfg.anchor_stride, block=cfg.block, grid=cfg.grid)
        torch.cuda.synchronize()
        ref_o, ref_l = _oracle_sparse(cfg, q, k, v, mask, rep, cfg.anchor_stride)
        assert_close_out(to_host(o)[0], ref_o, "f32", f"tiny sparse fuse={fuse}")
        assert_close_lse(to_host(lse)[0], ref_l, "tiny sparse", 1e-5)


def test_tiny_tau_one_is_dense(tiny):
    cfg, calib, (q, k, v) = tiny
    qc = np.stack([c[0] for c in calib])
    kc = np.stack([c[1] for c in calib])
    energy, _, _ = cba.calib_block_energy(torch.from_numpy(qc).cuda(), torch.from_numpy(kc).cuda(), None,
                                          block=cfg.block)
    mask = cba.select_blocks_by_energy(energy, 1.0, cfg.rho)
    assert bool(mask.bool().all())
    row_ptr, col_idx, order = cba.build_block_csr(mask)
    qd, kd, vd = to_dev(q, "f32"), to_dev(k, "f32"), to_dev(v, "f32")
    o = cba.sparse_attn_fwd(qd, kd, vd, row_ptr, col_idx, block=cfg.block, work_order=order)
    od = cba.dense_attn_fwd(qd, kd, vd, block=cfg.block)
    torch.cuda.synchronize()
    assert torch.equal(o, od)


# ---------------------------------------------------------------- selection / CSR / broadcast (exact)

@pytest.mark.parametrize("draws,heads,nb,tau,rho,prefix", [
    (3, 2, 8, 0.9, 0.5, 0), (4, 3, 70, 0.95, 0.5, 2), (1, 1, 5, 0.5, 0.5, 0), (2, 2, 33, 1.0, 0.5, 0),
    (4, 2, 591, 0.95, 0.5, 0), (4, 1, 929, 0.9, 0.49, 2), (1, 1, 4096, 0.95, 0.5, 0)])  # nb = 4096: the maximum
def test_select_bitexact_on_same_energy(draws, heads, nb, tau, rho, prefix):
    rng = np.random.default_rng(nb * 7 + draws)
    e = (rng.random((draws, heads, nb, nb)) ** 6).astype(np.float32)
    e[..., : nb // 3] = np.floor(e[..., : nb // 3] * 4) / 4  # exact ties (incl. zeros)
    ed = torch.from_numpy(e).cuda()
    mask, votes = cba.select_blocks_by_energy(ed, tau, rho, True, prefix, return_votes=True)
    torch.cuda.synchronize()
    m_ref, v_ref = oracle.select_blocks(e, tau, rho, True, prefix)
    np.testing.assert_array_equal(votes.cpu().numpy(), v_ref)
    np.testing.assert_array_equal(mask.cpu().numpy(), m_ref)


@pytest.mark.parametrize("rows,nkb,p", [(1, 1, 1.0), (16, 8, 0.4), (40, 591, 0.35), (300, 65, 0.5),
                                        (7, 64, 0.0), (24, 929, 0.9), (1000, 129, 0.05), (6, 65535, 0.3)])
def test_csr_bitexact(rows, nkb, p):
    rng = np.random.default_rng(rows + nkb)
    mask = (rng.random((rows, nkb)) < p).astype(np.uint8)
    if rows > 3:
        mask[2] = 0
        mask[3] = 1
    md = torch.from_numpy(mask).cuda()
    rp_ref, ci_ref, wo_ref = oracle.build_csr(mask)
    for exact in (False, True):
        rp, ci, wo = cba.build_block_csr(md, exact=exact)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(rp.cpu().numpy(), rp_ref)
        nnz = int(rp_ref[-1])
        np.testing.assert_array_equal(ci.cpu().numpy()[:nnz], ci_ref)
        np.testing.assert_array_equal(wo.cpu().numpy(), wo_ref)


def test_csr_capacity_guard():
    mask = np.ones((4, 10), dtype=np.uint8)
    md = torch.from_numpy(mask).cuda()
    rp = torch.empty(5, dtype=torch.int32, device="cuda")
    ci = torch.full((32,), -7, dtype=torch.int32, device="cuda")
    lib = cba.load_library()
    import ctypes
    st = lib.build_block_csr(ctypes.c_void_p(md.data_ptr()), 4, 10, ctypes.c_void_p(rp.data_ptr()),
                             ctypes.c_void_p(ci.data_ptr()), 25, None,
                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert st == 0
    assert int(rp[-1]) == 40  # the caller sees nnz > capacity
    got = ci.cpu().numpy()
    np.testing.assert_array_equal(got[:25], np.tile(np.arange(10), 3)[:25])
    assert (got[25:] == -7).all()  # nothing written past the capacity


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_broadcast_bitexact(dtype):
    cfg = _small_cfg(128, 128, (3, 10, 12), 128, dtype=dtype, heads=4)
    rng = np.random.default_rng(5)
    o = rng.standard_normal((4, cfg.seq_len, 128)).astype(np.float32)
    od = to_dev(o, dtype)
    base = to_host(od)[0]
    rep = np.array([1, 0, 1, 0], dtype=np.uint8)
    cba.rep_row_broadcast(od, rep, 3, block=128, n_prefix=128, grid=cfg.grid)
    torch.cuda.synchronize()
    got = to_host(od)[0]
    for h in range(4):
        ref = oracle.row_broadcast(base[h], 128, cfg.grid, 3) if rep[h] else base[h]
        np.testing.assert_array_equal(got[h], ref)


def test_deterministic_repeat():
    cfg = _small_cfg(128, 128, (2, 17, 20), 0)
    q, k, v = make_qkv(cfg, draw=0)
    mask = random_block_mask(cfg)
    row_ptr, col_idx, order = cba.build_block_csr(torch.from_numpy(mask).cuda())
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    a = cba.sparse_attn_fwd(qd, kd, vd, row_ptr, col_idx, block=128, work_order=order)
    b = cba.sparse_attn_fwd(qd, kd, vd, row_ptr, col_idx, block=128, work_order=None)
    e1, _, _ = cba.calib_block_energy(qd, kd, None, block=128)
    e2, _, _ = cba.calib_block_energy(qd, kd, None, block=128)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(e1, e2)


def test_wide_row_stride_takes_global_load_path():
    """Row strides so wide that a head's K/V rows need byte offsets beyond 31 bits
    send every kernel down its global-load path (clamped rows instead of a
    bounded buffer).  Same results, bit for bit, as the compact layout; the
    compact layout itself is checked against the oracle above."""
    cfg = _small_cfg(128, 128, (2, 17, 20), 0, heads=2)
    n, d = cfg.seq_len, cfg.head_dim
    sn = ((1 << 31) // (2 * (n + 64)) // 8 + 1) * 8  # (n + 64) * sn * 2 bytes >= 2^31
    log(f"wide stride: n={n} stride_n={sn} ({2 * n * sn * cfg.heads / 2**30:.1f} GiB per tensor)")
    q, k, v = make_qkv(cfg, draw=0)
    mask = random_block_mask(cfg)
    rep = rep_head_flags(cfg)
    row_ptr, col_idx, _ = cba.build_block_csr(torch.from_numpy(mask).cuda())
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")

    def wide(t):
        w = torch.zeros((1, cfg.heads, n, sn), dtype=t.dtype, device=t.device)[..., :d]
        w.copy_(t)
        return w

    qw, kw, vw = wide(qd), wide(kd), wide(vd)
    assert qw.stride(2) == sn
    ow = wide(torch.zeros_like(qd))
    kwargs = dict(block=128, rep_heads=rep, anchor_stride=4, grid=cfg.grid)
    o_c, l_c = cba.sparse_attn_fwd(qd, kd, vd, row_ptr, col_idx, return_lse=True, **kwargs)
    o_w, l_w = cba.sparse_attn_fwd(qw, kw, vw, row_ptr, col_idx, o=ow, return_lse=True, **kwargs)
    iv_ptr, ivs = cba.build_block_intervals(torch.from_numpy(mask).cuda())
    o_wi = cba.sparse_attn_fwd_intervals(qw, kw, vw, iv_ptr, ivs, o=wide(torch.zeros_like(qd)), **kwargs)
    e_c, le_c, _ = cba.calib_block_energy(qd, kd, None, block=128)
    e_w, le_w, _ = cba.calib_block_energy(qw, kw, None, block=128)
    d_c = cba.dense_attn_fwd(qd, kd, vd, block=128)
    d_w = cba.dense_attn_fwd(qw, kw, vw, block=128, o=wide(torch.zeros_like(qd)))
    torch.cuda.synchronize()
    assert torch.equal(o_c, o_w.contiguous()) and torch.equal(l_c, l_w)
    assert torch.equal(o_c, o_wi.contiguous())
    assert torch.equal(e_c, e_w) and torch.equal(le_c, le_w)
    assert torch.equal(d_c, d_w.contiguous())
    ref_o, _ = _oracle_sparse(cfg, q, k, v, mask, rep, 4)
    assert_close_out(to_host(o_w)[0], ref_o, "bf16", "wide-stride sparse O")
    del qw, kw, vw, ow, o_wi
    torch.cuda.empty_cache()


@pytest.mark.parametrize("factor", [0.0, 1.6, 2.0, 1e9])
def test_heavy_first_order_bitexact(factor):
    """order_heavy_rows_first against the oracle: the hand-derived counts, and a mask
    with two dense rows per head (like text tokens) over random sparse rows."""
    g_counts = np.array([3, 9, 2, 3, 12, 3, 0, 8])
    hand = (np.arange(12)[None, :] < g_counts[:, None]).astype(np.uint8)
    rng = np.random.default_rng(17)
    m = (rng.random((6 * 50, 50)) < 0.15).astype(np.uint8)
    m[::50] = 1
    m[1::50] = 1
    for mask in (hand, m):
        row_ptr, _, lpt = cba.build_block_csr(torch.from_numpy(mask).cuda())
        got = cba.order_heavy_rows_first(row_ptr, mask.shape[1], factor)
        torch.cuda.synchronize()
        ref = oracle.heavy_first_order(mask.sum(axis=1), factor)
        np.testing.assert_array_equal(got.cpu().numpy(), ref)
        if factor == 0.0:
            assert torch.equal(got, lpt)


def test_graph_capture_replays_match_eager():
    """The calls allocate nothing and take the caller's stream, so a HIP graph can
    capture them: skip-list build, sparse attention with a repetition head and the
    separate broadcast, replayed several times with eager work in between; every
    replay equals the eager result."""
    cfg = _small_cfg(128, 64, (2, 8, 16), 0, heads=2)
    q, k, v = make_qkv(cfg, draw=0)
    mask = random_block_mask(cfg)
    rep = rep_head_flags(cfg)
    qd, kd, vd = to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16")
    md = torch.from_numpy(mask).cuda()
    nb = cfg.nb
    row_ptr = torch.empty(cfg.heads * nb + 1, dtype=torch.int32, device="cuda")
    col_idx = torch.empty(cfg.heads * nb * nb, dtype=torch.int32, device="cuda")
    order = torch.empty(cfg.heads * nb, dtype=torch.int32, device="cuda")
    o = torch.zeros_like(qd)
    import ctypes
    lib = cba.load_library()
    desc = cba.make_desc(qd, cfg.block, 0, cfg.grid)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    rep_arr = np.ascontiguousarray(rep)

    def work():
        S = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        assert lib.build_block_csr(P(md), cfg.heads * nb, nb, P(row_ptr), P(col_idx), col_idx.numel(), P(order),
                                   S) == 0
        assert lib.sparse_attn_fwd(ctypes.byref(desc), P(qd), P(kd), P(vd), P(row_ptr), P(col_idx), col_idx.numel(),
                                   P(order), rep_arr.ctypes.data_as(ctypes.c_void_p), cfg.anchor_stride, 0, P(o),
                                   None, S) == 0
        assert lib.rep_row_broadcast(ctypes.byref(desc), P(o), rep_arr.ctypes.data_as(ctypes.c_void_p),
                                     cfg.anchor_stride, S) == 0

    work()
    torch.cuda.synchronize()
    eager = o.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()  # warm-up on the side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for rep_i in range(4):
        o.zero_()
        row_ptr.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, eager), f"replay {rep_i} differs"
        work()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(o, eager)
