"""Pins of the fp64 oracle against things other than itself: hand-derived worked
examples (tests/golden/hand_examples.json), a library routine (torch's CPU
scaled_dot_product_attention in fp64, torch.softmax), closed forms, invariants and
brute force over subsets.  CPU only."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")))


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sdpa(q, k, v, scale, mask=None):
    """torch's CPU fp64 SDPA; mask is a bool [N, N] (True = attend)."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64))[None, None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m, scale=scale)
    return o[0, 0].numpy()


# ---------------------------------------------------------------- dense attention

@pytest.mark.parametrize("n,d,seed", [(7, 4, 0), (64, 16, 1), (100, 32, 2)])
def test_dense_matches_library_sdpa(n, d, seed):
    q, k, v = _rand((n, d), seed), _rand((n, d), seed + 10), _rand((n, d), seed + 20)
    o, lse = oracle.dense_attention(q, k, v)
    ref = _sdpa(q, k, v, 1.0 / math.sqrt(d))
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
    s = torch.from_numpy(q @ k.T / math.sqrt(d))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=1).numpy(), rtol=0, atol=1e-12)


def test_dense_closed_forms():
    n, d = 37, 8
    v = _rand((n, d), 3)
    # Q = 0: every logit is 0, the softmax is uniform, o_i = mean_j v_j, LSE = ln N.
    o, lse = oracle.dense_attention(np.zeros((n, d)), _rand((n, d), 4), v)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(0), o.shape), atol=1e-13)
    np.testing.assert_allclose(lse, math.log(n), atol=1e-13)
    # constant V: convex weights reproduce the constant row.
    c = _rand((1, d), 5)
    o, _ = oracle.dense_attention(_rand((n, d), 6), _rand((n, d), 7), np.repeat(c, n, 0))
    np.testing.assert_allclose(o, np.repeat(c, n, 0), atol=1e-13)


def test_dense_lse_matches_scipy_logsumexp():
    """The LSE against scipy's logsumexp of the scaled logits (a second library)."""
    from scipy.special import logsumexp

    for n, d, seed in ((9, 4, 30), (80, 16, 31)):
        q, k, v = _rand((n, d), seed), 3.0 * _rand((n, d), seed + 1), _rand((n, d), seed + 2)
        _, lse = oracle.dense_attention(q, k, v)
        np.testing.assert_allclose(lse, logsumexp(q @ k.T / math.sqrt(d), axis=1), rtol=0, atol=1e-12)


def test_dense_shift_invariance():
    """Adding one vector u to every key adds scale * q_i . u to every logit of row i:
    the softmax of each row is unchanged (so O is), and the LSE moves by exactly that
    per-row constant.  A softmax over the wrong axis, or a dropped max shift, fails."""
    n, d = 30, 8
    q, k, v = _rand((n, d), 40), _rand((n, d), 41), _rand((n, d), 42)
    u = 4.0 * _rand((1, d), 43)
    o0, lse0 = oracle.dense_attention(q, k, v)
    o1, lse1 = oracle.dense_attention(q, k + u, v)
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse1 - lse0, (q @ u[0]) / math.sqrt(d), rtol=0, atol=1e-11)


def test_dense_explicit_scale():
    q, k, v = _rand((20, 8), 8), _rand((20, 8), 9), _rand((20, 8), 10)
    o, _ = oracle.dense_attention(q, k, v, scale=0.37)
    np.testing.assert_allclose(o, _sdpa(q, k, v, 0.37), atol=1e-12)


# ---------------------------------------------------------------- hand example

def _hand():
    g = GOLD["softmax_example"]
    q = np.array(g["q"])[:, None]
    k = np.log(np.array(g["k_exp"]))[:, None]
    v = np.array(g["v"])[:, None]
    return g, q, k, v


def test_hand_example_dense_energy_select_sparse():
    g, q, k, v = _hand()
    o, lse = oracle.dense_attention(q, k, v, scale=g["scale"])
    np.testing.assert_allclose(o[:, 0], g["dense_o"], atol=1e-12)
    np.testing.assert_allclose(lse, math.log(g["dense_lse_exp"]), atol=1e-12)
    e = oracle.block_energy(q, k, g["block"], scale=g["scale"])
    np.testing.assert_allclose(e, g["energy"], atol=1e-12)
    for tau, key in ((0.5, "keep_tau_0.5"), (0.75, "keep_tau_0.75")):
        keep = np.array([oracle.select_row(e[r], tau) for r in range(2)])
        np.testing.assert_array_equal(keep.astype(int), g[key])
    mask, votes = oracle.select_blocks(e[None, None], 0.5, rho=0.5, force_diag=True)
    np.testing.assert_array_equal(mask[0], g["mask_tau_0.5_forced_diag"])
    o, lse = oracle.sparse_attention(q, k, v, np.array(g["sparse_mask"]), g["block"], scale=g["scale"])
    np.testing.assert_allclose(o[:, 0], g["sparse_o_num"] / g["sparse_o_den"], atol=1e-12)
    np.testing.assert_allclose(lse, math.log(g["sparse_lse_exp"]), atol=1e-12)


def test_hand_selection_cases():
    for case in GOLD["selection_examples"]["cases"]:
        keep = oracle.select_row(np.array(case["e"], dtype=np.float64), case["tau"])
        np.testing.assert_array_equal(keep.astype(int), case["keep"], err_msg=str(case))


def test_hand_aggregation_cases():
    for case in GOLD["aggregation_example"]["cases"]:
        keep = oracle.aggregate_votes(np.array(case["votes"]), case["n_draws"], case["rho"])
        np.testing.assert_array_equal(keep.astype(int), case["keep"])


def test_hand_csr_case():
    g = GOLD["csr_example"]
    row_ptr, col_idx, order = oracle.build_csr(np.array(g["mask"], dtype=np.uint8))
    np.testing.assert_array_equal(row_ptr, g["row_ptr"])
    np.testing.assert_array_equal(col_idx, g["col_idx"])
    np.testing.assert_array_equal(order, g["work_order"])


def test_hand_interval_case():
    g = GOLD["interval_example"]
    iv_ptr, first, count, order = oracle.build_intervals(np.array(g["mask"], dtype=np.uint8))
    np.testing.assert_array_equal(iv_ptr, g["iv_ptr"])
    np.testing.assert_array_equal(first, g["first"])
    np.testing.assert_array_equal(count, g["count"])
    np.testing.assert_array_equal(order, g["work_order"])


def test_hand_broadcast_case():
    g = GOLD["broadcast_example"]
    n = g["n_prefix"] + int(np.prod(g["grid"]))
    o = np.arange(n, dtype=np.float64)[:, None] * np.ones((1, 3))
    out = oracle.row_broadcast(o, g["n_prefix"], g["grid"], g["stride"])
    np.testing.assert_array_equal(out[:, 0], g["source_token"])
    rows = oracle.computed_rows(n, g["n_prefix"], g["grid"], g["stride"], True)
    np.testing.assert_array_equal(rows.astype(int), g["computed_rows"])


# ---------------------------------------------------------------- block energy

@pytest.mark.parametrize("n,block", [(64, 16), (70, 16), (33, 8)])
def test_energy_matches_library_softmax_tiles(n, block):
    d = 8
    q, k = _rand((n, d), 11), _rand((n, d), 12)
    e = oracle.block_energy(q, k, block)
    p = torch.softmax(torch.from_numpy(q @ k.T / math.sqrt(d)), dim=1).numpy()
    nb = (n + block - 1) // block
    ref = np.zeros((nb, nb))
    for i in range(n):  # brute force: visit every probability once
        for j in range(n):
            ref[i // block, j // block] += p[i, j]
    np.testing.assert_allclose(e, ref, atol=1e-12)


@pytest.mark.parametrize("n,block", [(64, 16), (70, 16)])
def test_energy_invariants(n, block):
    d = 8
    q, k = _rand((n, d), 13) * 3, _rand((n, d), 14)
    e = oracle.block_energy(q, k, block)
    sizes = np.array([min(n, (b + 1) * block) - b * block for b in range((n + block - 1) // block)])
    assert (e >= 0).all()
    # each query row's probabilities sum to 1, so a query block's energies sum to its row count
    np.testing.assert_allclose(e.sum(axis=1), sizes, atol=1e-12)
    # Q = 0: uniform attention, so E[qb, kb] = |qb| * |kb| / N exactly (up to rounding)
    e0 = oracle.block_energy(np.zeros((n, d)), k, block)
    np.testing.assert_allclose(e0, np.outer(sizes, sizes) / n, atol=1e-13)


def test_energy_q_blocks_subset():
    q, k = _rand((50, 8), 15), _rand((50, 8), 16)
    full = oracle.block_energy(q, k, 16)
    part = oracle.block_energy(q, k, 16, q_blocks=[3, 0])
    np.testing.assert_array_equal(part, full[[3, 0]])


# ---------------------------------------------------------------- selection

def _brute_force_keep(e, tau):
    """Smallest subset reaching tau * total; among those, the one whose sorted
    member list under (energy desc, index asc) is first."""
    nkb = len(e)
    total = sum(e)
    rank = sorted(range(nkb), key=lambda j: (-e[j], j))
    pos = {j: r for r, j in enumerate(rank)}
    for size in range(1, nkb + 1):
        best = None
        for sub in itertools.combinations(range(nkb), size):
            if sum(e[j] for j in sub) >= tau * total:
                key = sorted(pos[j] for j in sub)
                if best is None or key < best[0]:
                    best = (key, sub)
        if best is not None:
            keep = np.zeros(nkb, dtype=bool)
            keep[list(best[1])] = True
            return keep
    return np.ones(nkb, dtype=bool)


@pytest.mark.parametrize("seed", range(12))
def test_selection_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    nkb = int(rng.integers(1, 11))
    e = rng.integers(0, 6, size=nkb).astype(np.float64)  # integers: every partial sum is exact
    if e.sum() == 0:
        e[0] = 1.0
    for tau in (0.1, 0.37, 0.5, 0.8, 0.95, 0.999):
        keep = oracle.select_row(e, tau)
        np.testing.assert_array_equal(keep, _brute_force_keep(list(e), tau), err_msg=f"e={e} tau={tau}")


def test_selection_monotone_and_extremes():
    rng = np.random.default_rng(21)
    e = rng.random(40) ** 4
    prev = 0
    for tau in np.linspace(0.01, 0.999, 60):
        cnt = int(oracle.select_row(e, tau).sum())
        assert cnt >= prev
        prev = cnt
    assert oracle.select_row(e, 1.0).all()
    tiny = oracle.select_row(e, 1e-9)
    assert tiny.sum() == 1 and tiny[np.argmax(e)]


def test_aggregation_identities():
    rng = np.random.default_rng(22)
    e = rng.random((1, 3, 6, 6))
    # one draw: the aggregated mask is that draw's selection
    mask, votes = oracle.select_blocks(e, 0.8, rho=0.5, force_diag=False)
    for h in range(3):
        for r in range(6):
            np.testing.assert_array_equal(mask[h, r].astype(bool), oracle.select_row(e[0, h, r], 0.8))
    # identical draws: same mask, every vote equals the draw count or 0
    mask4, votes4 = oracle.select_blocks(np.repeat(e, 4, axis=0), 0.8, rho=0.5, force_diag=False)
    np.testing.assert_array_equal(mask4, mask)
    assert set(np.unique(votes4)) <= {0, 4}


def test_forced_blocks():
    e = np.zeros((2, 1, 5, 5))
    e[..., 4] = 1.0  # all energy in the last key block
    mask, _ = oracle.select_blocks(e, 0.5, rho=0.5, force_diag=True, n_dense_prefix_blocks=2)
    m = mask[0].astype(bool)
    assert m[np.arange(5), np.arange(5)].all()
    assert m[:2, :].all() and m[:, :2].all() and m[:, 4].all()
    assert not m[2, 3] and not m[3, 2]


def test_tau_one_calibration_gives_dense_output():
    n, d, block = 48, 8, 16
    q, k, v = _rand((n, d), 23), _rand((n, d), 24), _rand((n, d), 25)
    e = oracle.block_energy(q, k, block)[None, None]
    mask, _ = oracle.select_blocks(e, 1.0)
    assert mask.all()
    o, lse = oracle.sparse_attention(q, k, v, mask[0], block)
    od, lsed = oracle.dense_attention(q, k, v)
    np.testing.assert_allclose(o, od, atol=1e-13)
    np.testing.assert_allclose(lse, lsed, atol=1e-13)


# ---------------------------------------------------------------- CSR

@pytest.mark.parametrize("seed", range(4))
def test_csr_round_trip(seed):
    rng = np.random.default_rng(seed)
    rows, nkb = int(rng.integers(1, 50)), int(rng.integers(1, 40))
    mask = (rng.random((rows, nkb)) < rng.random()).astype(np.uint8)
    row_ptr, col_idx, order = oracle.build_csr(mask)
    back = np.zeros_like(mask)
    for r in range(rows):
        seg = col_idx[row_ptr[r]:row_ptr[r + 1]]
        assert (np.diff(seg) > 0).all()
        back[r, seg] = 1
    np.testing.assert_array_equal(back, mask)
    assert row_ptr[-1] == mask.sum()
    assert sorted(order.tolist()) == list(range(rows))
    cnt = np.diff(row_ptr)[order]
    assert (np.diff(cnt) <= 0).all()
    for a, b in zip(order[:-1], order[1:]):  # equal counts keep row order
        if cnt[list(order).index(a)] == cnt[list(order).index(b)]:
            assert a < b


# ---------------------------------------------------------------- sparse attention

@pytest.mark.parametrize("n,block,density,seed", [(64, 16, 0.4, 0), (70, 16, 0.5, 1), (96, 32, 0.3, 2)])
def test_sparse_matches_library_masked_sdpa(n, block, density, seed):
    d = 8
    rng = np.random.default_rng(seed)
    q, k, v = _rand((n, d), 30 + seed), _rand((n, d), 40 + seed), _rand((n, d), 50 + seed)
    nb = (n + block - 1) // block
    m = rng.random((nb, nb)) < density
    np.fill_diagonal(m, True)
    o, lse = oracle.sparse_attention(q, k, v, m, block)
    tok = oracle.token_mask_from_blocks(m, block, n)
    np.testing.assert_allclose(o, _sdpa(q, k, v, 1 / math.sqrt(d), tok), atol=1e-12)
    s = torch.from_numpy(q @ k.T / math.sqrt(d)).masked_fill(~torch.from_numpy(tok), -math.inf)
    np.testing.assert_allclose(lse, torch.logsumexp(s, 1).numpy(), atol=1e-12)


def test_token_mask_expansion_by_hand():
    m = np.array([[1, 0], [0, 1]], dtype=bool)
    t = oracle.token_mask_from_blocks(m, 2, 3)
    np.testing.assert_array_equal(t, [[1, 1, 0], [1, 1, 0], [0, 0, 1]])


def test_sparse_full_mask_is_dense_and_diagonal_is_blockwise():
    n, d, block = 80, 8, 16
    q, k, v = _rand((n, d), 60), _rand((n, d), 61), _rand((n, d), 62)
    nb = n // block
    o, lse = oracle.sparse_attention(q, k, v, np.ones((nb, nb)), block)
    od, lsed = oracle.dense_attention(q, k, v)
    np.testing.assert_allclose(o, od, atol=1e-13)
    o, _ = oracle.sparse_attention(q, k, v, np.eye(nb), block)
    for b in range(nb):
        sl = slice(b * block, (b + 1) * block)
        np.testing.assert_allclose(o[sl], _sdpa(q[sl], k[sl], v[sl], 1 / math.sqrt(d)), atol=1e-12)


def test_sparse_masked_values_change_nothing():
    """For the rows of one query block, the V and K rows of key blocks outside its
    mask take no part: perturbing them (even by huge values) leaves those rows'
    outputs and LSE bit-identical.  Masking by a zero weight after the softmax, or
    over the wrong block row, fails."""
    n, d, block = 96, 8, 16
    nb = n // block
    q, k, v = _rand((n, d), 50), _rand((n, d), 51), _rand((n, d), 52)
    rng = np.random.default_rng(53)
    mask = rng.random((nb, nb)) < 0.4
    np.fill_diagonal(mask, True)
    for qb in range(nb):
        rows = np.zeros(n, dtype=bool)
        rows[qb * block:(qb + 1) * block] = True
        o0, lse0 = oracle.sparse_attention(q, k, v, mask, block, rows=rows)
        k2, v2 = k.copy(), v.copy()
        for kb in np.nonzero(~mask[qb])[0]:
            k2[kb * block:(kb + 1) * block] += 1e3 * _rand((block, d), 54 + kb)
            v2[kb * block:(kb + 1) * block] = 1e6 * _rand((block, d), 70 + kb)
        o1, lse1 = oracle.sparse_attention(q, k2, v2, mask, block, rows=rows)
        np.testing.assert_array_equal(o1[rows], o0[rows])
        np.testing.assert_array_equal(lse1[rows], lse0[rows])


def test_sparse_empty_rows_and_row_subset():
    n, d, block = 48, 4, 16
    q, k, v = _rand((n, d), 63), _rand((n, d), 64), _rand((n, d), 65)
    m = np.ones((3, 3), dtype=bool)
    m[1] = False
    o, lse = oracle.sparse_attention(q, k, v, m, block)
    assert (o[16:32] == 0).all() and np.isneginf(lse[16:32]).all()
    full, _ = oracle.sparse_attention(q, k, v, np.ones((3, 3)), block)
    rows = np.array([0, 5, 40, 47])
    part, lp = oracle.sparse_attention(q, k, v, np.ones((3, 3)), block, rows=rows)
    np.testing.assert_array_equal(part[rows], full[rows])
    others = np.setdiff1d(np.arange(n), rows)
    assert (part[others] == 0).all() and np.isneginf(lp[others]).all()


# ---------------------------------------------------------------- repetition

def test_broadcast_stride_one_is_identity():
    o = _rand((2 + 3 * 4 * 5, 6), 70)
    np.testing.assert_array_equal(oracle.row_broadcast(o, 2, (3, 4, 5), 1), o)
    assert oracle.computed_rows(o.shape[0], 2, (3, 4, 5), 1, True).all()


def test_repetition_equals_full_computation_when_rows_repeat():
    # Each group of s image rows repeats its anchor row's queries, and the grid is
    # laid out so a group never straddles a query block (W*s == block): then the
    # anchors' outputs are exactly every row's output.
    grid, s, block, n_prefix = (3, 8, 4), 2, 8, 8
    n = n_prefix + 3 * 8 * 4
    d = 8
    rng = np.random.default_rng(71)
    q = rng.standard_normal((n, d))
    g = q[n_prefix:].reshape(3, 8, 4, d)
    g[:, 1::2] = g[:, 0::2]
    q[n_prefix:] = g.reshape(-1, d)
    k, v = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    nb = n // block
    m = rng.random((nb, nb)) < 0.5
    np.fill_diagonal(m, True)
    full, lfull = oracle.sparse_attention(q, k, v, m, block)
    rep, lrep = oracle.sparse_attention_with_repetition(q, k, v, m, block, n_prefix, grid, s, True)
    np.testing.assert_allclose(rep, full, atol=1e-13)
    np.testing.assert_allclose(lrep, lfull, atol=1e-13)
    # a normal head computes every row
    nrm, _ = oracle.sparse_attention_with_repetition(q, k, v, m, block, n_prefix, grid, s, False)
    np.testing.assert_array_equal(nrm, full)


def test_repetition_short_last_group():
    # H = 5 with s = 4: anchors 0 and 4; row 4 stands only for itself.
    rows = oracle.computed_rows(1 * 5 * 3, 0, (1, 5, 3), 4, True)
    np.testing.assert_array_equal(rows.reshape(5, 3)[:, 0], [1, 0, 0, 0, 1])
    o = np.arange(15, dtype=np.float64)[:, None]
    out = oracle.row_broadcast(o, 0, (1, 5, 3), 4).reshape(5, 3)
    np.testing.assert_array_equal(out[:, 1], [1, 1, 1, 1, 13])


# ---------------------------------------------------------------- repetition detection


def _grid_pairs(n_prefix, grid, s):
    """(follower, anchor) tokens enumerated over (f, y, x) of the token grid."""
    f_, h_, w_ = grid
    fol, anc = [], []
    for f in range(f_):
        for y in range(h_):
            if y % s == 0:
                continue
            for x in range(w_):
                fol.append(n_prefix + (f * h_ + y) * w_ + x)
                anc.append(n_prefix + (f * h_ + (y // s) * s) * w_ + x)
    return np.array(fol), np.array(anc)


def test_hand_repetition_pairs():
    g = GOLD["repetition_pairs_example"]
    n = g["n_prefix"] + int(np.prod(g["grid"]))
    rng = np.random.default_rng(80)
    q, k = rng.standard_normal((n, 6)), rng.standard_normal((n, 6))
    toks, cos = oracle.repetition_cosines(q, k, g["n_prefix"], g["grid"], g["stride"])
    np.testing.assert_array_equal(toks, g["followers"])
    assert np.all(cos < 1 - 1e-6)  # distinct random queries: never identical rows
    # a follower whose query equals that of its hand-derived anchor attends identically
    q[g["followers"]] = q[g["anchors"]]
    _, cos = oracle.repetition_cosines(q, k, g["n_prefix"], g["grid"], g["stride"])
    np.testing.assert_allclose(cos, 1.0, atol=1e-13)


def test_hand_repetition_cosine():
    g = GOLD["repetition_cosine_example"]
    q = math.log(2.0) * np.array(g["q_units"], dtype=np.float64)
    k = np.eye(4)
    want = np.array(g["cos_num"]) / np.sqrt(np.array(g["cos_den_sq"], dtype=np.float64))
    toks, cos = oracle.repetition_cosines(q, k, g["n_prefix"], g["grid"], g["stride"], scale=g["scale"])
    np.testing.assert_array_equal(toks, g["followers"])
    np.testing.assert_allclose(cos, want, rtol=1e-14)
    score, full = oracle.repetition_score(q, k, g["n_prefix"], g["grid"], g["stride"], scale=g["scale"])
    assert abs(score - want.mean()) < 1e-14
    assert np.isnan(full[:2]).all() and np.allclose(full[2:], want, rtol=1e-14)


def _two_level_cos(n, key_group, set_a, set_b, beta):
    """Closed form of the cosine between two softmax rows whose logits are beta on
    the keys of some groups and 0 elsewhere: with weight w = e^beta, the
    unnormalised rows hold w or 1 and the normalisations cancel."""
    in_a, in_b = set_a[key_group], set_b[key_group]
    both = int(np.sum(in_a & in_b))
    one = int(np.sum(in_a ^ in_b))
    neither = n - int(np.sum(in_a | in_b))
    w = math.exp(beta)
    dot = both * w * w + one * w + neither
    na = int(in_a.sum()) * w * w + (n - int(in_a.sum()))
    nb = int(in_b.sum()) * w * w + (n - int(in_b.sum()))
    return dot / math.sqrt(na * nb)


@pytest.mark.parametrize("n_prefix,grid,s,seed", [(0, (2, 6, 5), 2, 81), (4, (3, 7, 4), 4, 82),
                                                  (2, (1, 9, 3), 3, 83)])
def test_repetition_two_level_closed_form(n_prefix, grid, s, seed):
    n = n_prefix + int(np.prod(grid))
    d, beta = 12, 1.7
    rng = np.random.default_rng(seed)
    key_group = rng.integers(0, d, n)
    k = np.eye(d)[key_group]
    sets = rng.random((n, d)) < 0.4
    q = beta * sets.astype(np.float64)
    toks, cos = oracle.repetition_cosines(q, k, n_prefix, grid, s, scale=1.0)
    fol, anc = _grid_pairs(n_prefix, grid, s)
    np.testing.assert_array_equal(toks, fol)
    want = np.array([_two_level_cos(n, key_group, sets[a], sets[i], beta) for i, a in zip(fol, anc)])
    np.testing.assert_allclose(cos, want, rtol=1e-13)
    score, _ = oracle.repetition_score(q, k, n_prefix, grid, s, scale=1.0)
    assert abs(score - want.mean()) < 1e-13
    # the default scale 1/sqrt(d) is the same as beta / sqrt(d)
    toks2, cos2 = oracle.repetition_cosines(q, k, n_prefix, grid, s)
    want2 = [_two_level_cos(n, key_group, sets[a], sets[i], beta / math.sqrt(d)) for i, a in zip(fol, anc)]
    np.testing.assert_allclose(cos2, want2, rtol=1e-13)


def test_repetition_invariants():
    n_prefix, grid, s = 3, (2, 5, 4), 2
    n = n_prefix + 40
    rng = np.random.default_rng(84)
    q, k = rng.standard_normal((n, 8)), rng.standard_normal((n, 8))
    toks, cos = oracle.repetition_cosines(q, k, n_prefix, grid, s)
    assert np.all((cos > 0) & (cos <= 1 + 1e-15))
    # probabilities do not change when every key is shifted by one vector (each row's
    # logits move by a constant) or when the keys are permuted
    _, c_shift = oracle.repetition_cosines(q, k + rng.standard_normal(8) * 3, n_prefix, grid, s)
    np.testing.assert_allclose(c_shift, cos, rtol=1e-12)
    _, c_perm = oracle.repetition_cosines(q, k[rng.permutation(n)], n_prefix, grid, s)
    np.testing.assert_allclose(c_perm, cos, rtol=1e-12)
    # equal keys: every row is uniform
    _, c_uni = oracle.repetition_cosines(q, np.ones((n, 8)), n_prefix, grid, s)
    np.testing.assert_allclose(c_uni, 1.0, atol=1e-14)
    # a subset of followers gives the same values
    pick = toks[::3]
    t_sub, c_sub = oracle.repetition_cosines(q, k, n_prefix, grid, s, tokens=pick)
    np.testing.assert_array_equal(t_sub, pick)
    np.testing.assert_array_equal(c_sub, cos[::3])
    with pytest.raises(ValueError):
        oracle.repetition_cosines(q, k, n_prefix, grid, s, tokens=[n_prefix])  # an anchor
    with pytest.raises(ValueError):
        oracle.repetition_cosines(q, k, n_prefix, grid, 1)
    with pytest.raises(ValueError):
        oracle.repetition_cosines(q[:n_prefix + 8], k[:n_prefix + 8], n_prefix, (2, 1, 4), 2)


def test_hand_repetition_flags():
    g = GOLD["repetition_flag_examples"]
    flags = oracle.mark_repetition_heads(np.array(g["scores"]), g["gamma"])
    np.testing.assert_array_equal(flags, g["flags"])
    assert flags.dtype == np.uint8
    # one draw: a plain strict threshold
    np.testing.assert_array_equal(oracle.mark_repetition_heads([[0.5, 0.25, 0.75]], 0.5), [0, 0, 1])


# ---------------------------------------------------------------- interval skip lists


@pytest.mark.parametrize("rows,nkb,density,seed", [(7, 1, 0.5, 90), (30, 13, 0.0, 91), (30, 13, 1.0, 92),
                                                   (50, 40, 0.3, 93), (20, 64, 0.8, 94)])
def test_intervals_round_trip_maximal_and_counted(rows, nkb, density, seed):
    m = np.random.default_rng(seed).random((rows, nkb)) < density
    iv_ptr, first, count, order = oracle.build_intervals(m)
    assert iv_ptr[0] == 0 and np.all(np.diff(iv_ptr) >= 0)
    back = np.zeros_like(m)
    for r in range(rows):
        runs = list(zip(first[iv_ptr[r]:iv_ptr[r + 1]], count[iv_ptr[r]:iv_ptr[r + 1]]))
        for (f0, c0), (f1, _) in zip(runs, runs[1:]):
            assert f1 > f0 + c0  # ascending, and a skipped block between two runs
        for f0, c0 in runs:
            assert c0 >= 1 and f0 + c0 <= nkb
            back[r, f0:f0 + c0] = True
        # brute force: one run per kept block whose left neighbour is skipped
        starts = sum(1 for c in range(nkb) if m[r, c] and (c == 0 or not m[r, c - 1]))
        assert len(runs) == starts
    np.testing.assert_array_equal(back, m)
    np.testing.assert_array_equal(order, oracle.build_csr(m)[2])


def test_intervals_of_a_band_are_few():
    # a band of width 5 around the diagonal is one run per row
    nkb = 20
    m = np.abs(np.arange(nkb)[:, None] - np.arange(nkb)[None, :]) <= 2
    iv_ptr, first, count, _ = oracle.build_intervals(m)
    np.testing.assert_array_equal(np.diff(iv_ptr), 1)
    np.testing.assert_array_equal(first, np.maximum(np.arange(nkb) - 2, 0))
    np.testing.assert_array_equal(count, m.sum(axis=1))


# ---------------------------------------------------------------- online search pieces


def test_hand_cached_lse_energy():
    g = GOLD["cached_lse_example"]
    h = GOLD["softmax_example"]
    q = np.array(h["q"])[:, None]
    k = np.log(np.array(h["k_exp"]))[:, None]
    lse = np.full(4, math.log(g["lse_uniform_exp"]))
    np.testing.assert_allclose(oracle.block_energy_from_lse(q, k, lse, h["block"], scale=h["scale"]),
                               g["energy_uniform"], rtol=1e-14)
    lse = np.log(np.array(g["lse_rows_exp"]))
    np.testing.assert_allclose(oracle.block_energy_from_lse(q, k, lse, h["block"], scale=h["scale"]),
                               g["energy_rows"], rtol=1e-14)


@pytest.mark.parametrize("n,block", [(96, 32), (77, 16)])
def test_energy_from_lse_against_block_energy(n, block):
    rng = np.random.default_rng(n)
    q, k, v = rng.standard_normal((n, 8)), rng.standard_normal((n, 8)), rng.standard_normal((n, 8))
    _, lse = oracle.dense_attention(q, k, v)
    ref = oracle.block_energy(q, k, block)
    np.testing.assert_allclose(oracle.block_energy_from_lse(q, k, lse, block), ref, rtol=1e-12)
    # a common shift scales every energy by exp(-shift)
    np.testing.assert_allclose(oracle.block_energy_from_lse(q, k, lse + 0.7, block), ref * math.exp(-0.7),
                               rtol=1e-12)
    # per-row shifts: each query block's total is the sum of its rows' exp(-shift)
    delta = rng.uniform(-1, 1, n)
    e = oracle.block_energy_from_lse(q, k, lse + delta, block)
    totals = [np.exp(-delta[qb * block:(qb + 1) * block]).sum() for qb in range(e.shape[0])]
    np.testing.assert_allclose(e.sum(axis=1), totals, rtol=1e-12)
    sub = oracle.block_energy_from_lse(q, k, lse, block, q_blocks=[1, 0])
    np.testing.assert_array_equal(sub, oracle.block_energy_from_lse(q, k, lse, block)[[1, 0]])


def test_hand_per_head_tau_selection():
    g = GOLD["per_head_tau_example"]
    e = np.array(g["e"], dtype=np.float64)
    energy = np.stack([e, e])[None, :, None, :]  # [draws 1, heads 2, rows 1, nkb]
    mask, _ = oracle.select_blocks(energy, g["tau"], rho=0.5, force_diag=False)
    np.testing.assert_array_equal(mask[:, 0], g["keep"])
    # equal per-head thresholds are the scalar threshold
    rng = np.random.default_rng(5)
    en = rng.random((3, 4, 6, 6))
    a, va = oracle.select_blocks(en, [0.8] * 4, 0.5)
    b, vb = oracle.select_blocks(en, 0.8, 0.5)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(va, vb)


def test_hand_heavy_first_order():
    g = GOLD["heavy_first_example"]
    for f in ("1.5", "1.6", "2", "3"):
        np.testing.assert_array_equal(oracle.heavy_first_order(g["counts"], float(f)), g["order_" + f])


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_heavy_first_order_limits(seed):
    rng = np.random.default_rng(seed)
    m = rng.random((60, 30)) < rng.uniform(0.05, 0.9, (60, 1))
    counts = m.sum(axis=1)
    for f in (0.5, 1.0, 1.7):
        order = oracle.heavy_first_order(counts, f)
        assert sorted(order.tolist()) == list(range(60))  # a permutation
    # factor 0: every row with a kept block is heavy, so the order is longest-first
    np.testing.assert_array_equal(oracle.heavy_first_order(counts, 0.0), oracle.build_csr(m)[2])
    # a factor no row reaches leaves the natural order
    np.testing.assert_array_equal(oracle.heavy_first_order(counts, 1e9), np.arange(60))
