"""Planted mistakes in the fp64 oracle (CPU only), used to show that the oracle's
pins in test_oracle.py catch plausible errors.  Each mutant replaces one oracle
function with a subtly wrong version; tests/test_oracle_mutations.py runs the pin
suite once per mutant and expects it to fail."""
import math

import numpy as np

from oracle import calibattn_oracle as O

_orig = {name: getattr(O, name) for name in dir(O) if not name.startswith("__")}


def _softmax_rows(s):
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    return e / l, (m + np.log(l))[:, 0]


def dense_no_scale(q, k, v, scale=None):
    return _orig["dense_attention"](q, k, v, scale=1.0)


def dense_softmax_over_queries(q, k, v, scale=None):
    q, k, v = O._f64(q), O._f64(k), O._f64(v)
    c = O._scale(q.shape[1], scale)
    s = (q @ k.T) * c
    p, _ = _softmax_rows(s.T)
    _, lse = _softmax_rows(s)
    return p.T @ v, lse


def energy_transposed(q, k, block, scale=None, q_blocks=None):
    full = _orig["block_energy"](q, k, block, scale)
    t = full.T
    return t if q_blocks is None else t[list(q_blocks)]


def energy_mean_not_sum(q, k, block, scale=None, q_blocks=None):
    e = _orig["block_energy"](q, k, block, scale, q_blocks)
    return e / float(block * block)


def select_ties_high_index_first(e, tau):
    e = O._f64(e)
    nkb = e.shape[0]
    keep = np.zeros(nkb, dtype=bool)
    if tau >= 1.0:
        keep[:] = True
        return keep
    order = np.lexsort((-np.arange(nkb), -e))
    run = np.cumsum(e[order])
    k = int(np.argmax(run >= tau * run[-1])) + 1
    keep[order[:k]] = True
    return keep


def select_strict_threshold(e, tau):
    e = O._f64(e)
    nkb = e.shape[0]
    keep = np.zeros(nkb, dtype=bool)
    if tau >= 1.0:
        keep[:] = True
        return keep
    order = np.lexsort((np.arange(nkb), -e))
    run = np.cumsum(e[order])
    hit = run > tau * run[-1]
    k = int(np.argmax(hit)) + 1 if hit.any() else nkb
    keep[order[:k]] = True
    return keep


def select_lowest_energy_first(e, tau):
    e = O._f64(e)
    nkb = e.shape[0]
    keep = np.zeros(nkb, dtype=bool)
    if tau >= 1.0:
        keep[:] = True
        return keep
    order = np.lexsort((np.arange(nkb), e))
    run = np.cumsum(e[order])
    k = int(np.argmax(run >= tau * run[-1])) + 1
    keep[order[:k]] = True
    return keep


def aggregate_at_least(votes, n_draws, rho):
    return np.asarray(votes) >= (float(rho) * float(n_draws))


def csr_unstable_order(mask):
    row_ptr, col_idx, _ = _orig["build_csr"](mask)
    counts = np.diff(row_ptr)
    order = np.lexsort((-np.arange(counts.size), -counts)).astype(np.int32)
    return row_ptr, col_idx, order


def sparse_masked_as_zero_logits(q, k, v, mask_h, block, scale=None, rows=None):
    """Skipped blocks take part with logit 0 instead of being excluded."""
    q, k, v = O._f64(q), O._f64(k), O._f64(v)
    n, d = q.shape
    c = O._scale(d, scale)
    tok = O.token_mask_from_blocks(mask_h, block, n)
    s = np.where(tok, (q @ k.T) * c, 0.0)
    p, lse = _softmax_rows(s)
    o = p @ v
    if rows is not None:
        rows = np.asarray(rows)
        want = rows if rows.dtype == bool else np.isin(np.arange(n), rows)
        o[~want] = 0
        lse[~want] = -np.inf
    return o, lse


def broadcast_along_x(o, n_prefix, grid, anchor_stride):
    out = np.array(o, copy=True)
    f_, h_, w_ = grid
    s = int(anchor_stride)
    if s <= 1:
        return out
    g = out[n_prefix:n_prefix + f_ * h_ * w_].reshape(f_, h_, w_, -1)
    anchors = (np.arange(w_) // s) * s
    out[n_prefix:n_prefix + f_ * h_ * w_] = g[:, :, anchors].reshape(f_ * h_ * w_, -1)
    return out


def rows_wrong_anchor(seq_len, n_prefix, grid, anchor_stride, is_rep_head):
    rows = np.ones(seq_len, dtype=bool)
    if not is_rep_head:
        return rows
    f_, h_, w_ = grid
    t = np.arange(n_prefix, seq_len)
    y = ((t - n_prefix) // w_) % h_
    rows[n_prefix:] = (y % anchor_stride) == min(1, anchor_stride - 1)
    return rows


def pairs_previous_row(seq_len, n_prefix, grid, anchor_stride):
    """Each follower compared with the image row just above it."""
    follower, _ = _orig["_follower_anchor_pairs"](seq_len, n_prefix, grid, anchor_stride)
    return follower, follower - grid[2]


def rep_cosine_of_logits(q, k, n_prefix, grid, anchor_stride, scale=None, tokens=None):
    """Cosine of the score rows instead of the probability rows."""
    q, k = O._f64(q), O._f64(k)
    c = O._scale(q.shape[1], scale)
    follower, anchor = O._follower_anchor_pairs(q.shape[0], n_prefix, grid, anchor_stride)
    if int(anchor_stride) < 2 or follower.size == 0:
        raise ValueError("no followers")
    if tokens is not None:
        pos = np.searchsorted(follower, np.asarray(tokens))
        follower, anchor = follower[pos], anchor[pos]
    sf, sa = (q[follower] @ k.T) * c, (q[anchor] @ k.T) * c
    cos = (sf * sa).sum(1) / (np.linalg.norm(sf, axis=1) * np.linalg.norm(sa, axis=1))
    return follower, cos


def rep_score_counts_anchors(q, k, n_prefix, grid, anchor_stride, scale=None):
    """Anchor rows counted in the mean with similarity 1."""
    _, full = _orig["repetition_score"](q, k, n_prefix, grid, anchor_stride, scale)
    g = full[n_prefix:]
    return float(np.where(np.isnan(g), 1.0, g).mean()), full


def mark_any_draw(scores, gamma):
    return (np.asarray(scores) > gamma).any(axis=0).astype(np.uint8)


def mark_at_least(scores, gamma):
    return (np.asarray(scores, dtype=np.float64).mean(axis=0) >= gamma).astype(np.uint8)


def intervals_unmerged(mask):
    """Every kept block its own run."""
    row_ptr, col_idx, order = _orig["build_csr"](mask)
    return row_ptr, col_idx, np.ones_like(col_idx), order


def intervals_inclusive_end(mask):
    """Run length taken as (last - first + 1) of an exclusive end."""
    iv_ptr, first, count, order = _orig["build_intervals"](mask)
    return iv_ptr, first, count + 1, order


def energy_from_lse_recomputed(q, k, lse, block, scale=None, q_blocks=None):
    """Ignores the given LSE and renormalises each row."""
    return _orig["block_energy"](q, k, block, scale, q_blocks)


def select_first_head_tau(energy, tau, rho=0.5, force_diag=True, n_dense_prefix_blocks=0):
    """Uses the first head's threshold for every head."""
    return _orig["select_blocks"](energy, np.ravel(np.asarray(tau))[0], rho, force_diag, n_dense_prefix_blocks)


def heavy_first_at_least(counts, factor):
    """Rows equal to the threshold counted as heavy."""
    counts = np.asarray(counts, dtype=np.int64)
    thr = float(factor) * (float(counts.sum()) / float(counts.size))
    heavy = np.nonzero(counts >= thr)[0]
    heavy = heavy[np.argsort(-counts[heavy], kind="stable")]
    light = np.nonzero(counts < thr)[0]
    return np.concatenate([heavy, light]).astype(np.int32)


MUTANTS = {
    "dense_no_scale": ("dense_attention", dense_no_scale),
    "dense_softmax_over_queries": ("dense_attention", dense_softmax_over_queries),
    "energy_transposed": ("block_energy", energy_transposed),
    "energy_mean_not_sum": ("block_energy", energy_mean_not_sum),
    "select_ties_high_index_first": ("select_row", select_ties_high_index_first),
    "select_strict_threshold": ("select_row", select_strict_threshold),
    "select_lowest_energy_first": ("select_row", select_lowest_energy_first),
    "aggregate_at_least": ("aggregate_votes", aggregate_at_least),
    "csr_unstable_order": ("build_csr", csr_unstable_order),
    "sparse_masked_as_zero_logits": ("sparse_attention", sparse_masked_as_zero_logits),
    "broadcast_along_x": ("row_broadcast", broadcast_along_x),
    "rows_wrong_anchor": ("computed_rows", rows_wrong_anchor),
    "pairs_previous_row": ("_follower_anchor_pairs", pairs_previous_row),
    "rep_cosine_of_logits": ("repetition_cosines", rep_cosine_of_logits),
    "rep_score_counts_anchors": ("repetition_score", rep_score_counts_anchors),
    "mark_any_draw": ("mark_repetition_heads", mark_any_draw),
    "mark_at_least": ("mark_repetition_heads", mark_at_least),
    "intervals_unmerged": ("build_intervals", intervals_unmerged),
    "intervals_inclusive_end": ("build_intervals", intervals_inclusive_end),
    "energy_from_lse_recomputed": ("block_energy_from_lse", energy_from_lse_recomputed),
    "select_first_head_tau": ("select_blocks", select_first_head_tau),
    "heavy_first_at_least": ("heavy_first_order", heavy_first_at_least),
}


def apply(name):
    """Install mutant `name` in the oracle module and package namespace."""
    import oracle

    target, fn = MUTANTS[name]
    setattr(O, target, fn)
    setattr(oracle, target, fn)
