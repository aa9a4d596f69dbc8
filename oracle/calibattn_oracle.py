"""Plain, slow, fp64 CPU oracle of calibrated block-sparse spatiotemporal attention.

TEST INFRASTRUCTURE: imported only by the tests, the smoke check and the
benchmark's CPU-baseline leg.  It shares no code with the GPU library.

Sources (web summaries of two papers; cited by page and section):
  [CA-zh]  "Accelerating Text-to-Video Generation with Calibrated Sparse Attention
           (CalibAtt)", technical summary on gist.science (Chinese version):
           S1 problem, S2.1 observations, S2.2A offline calibration, S2.2B inference.
  [CA-de]  the German version, "Technische Zusammenfassung": S2A calibration,
           S2B inference.
  [CA-pt]  the Portuguese version, "Resumo tecnico": S2A, S2B.
  [CA-fr]  the French version, "Resume technique": S2A observations,
           S2B calibration, S2C inference.
  [AdaSpa] summary of "Training-free and Adaptive Sparse Attention for Efficient
           Long Video Generation" (ICCV 2025): S2 method.

Conventions shared by every function:
  * one head at a time: q, k, v are [N, d]; they are promoted to fp64 exactly;
  * scale defaults to 1/sqrt(d);
  * blocks are contiguous runs of `block` tokens in the frame-major token order;
    the last block is ragged when N is not a multiple of `block`;
  * a block mask is [nqb, nkb] with 1 = kept (the summaries' "skip list" lists the
    blocks that are computed).

Readings of points the pages leave open (each is repeated where it is used; R10-R16
concern block geometry, text tokens, the scale and encodings, which the functions
below take as parameters):
  R1 energy is the raw sum of attention probabilities over the B x B tile;
  R2 the threshold is a fraction of the query block's own total energy;
  R3 "reach" means cumulative energy >= tau * total;
  R4 equal energies are ordered by ascending key-block index;
  R5 tau >= 1 keeps every block;
  R6 aggregation keeps a block when its vote count is strictly above rho * draws;
  R7 the diagonal block, and the rows and columns of dense prefix (text) blocks,
     are forced kept after aggregation;
  R8 a "spatial row" is one image row (f, y) of W tokens; anchors are the rows with
     y mod s == 0 and each stands for rows y .. y+s-1 of its frame;
  R9 an anchor row keeps its own query block's mask; text tokens are never followers;
  R17 the "attention vector" of a token is its row of dense attention probabilities
     (softmax over all keys), and a follower token is compared with the token that
     the broadcast copies into it: its anchor, same frame and column;
  R18 a head's repetition score is the mean of those cosines over all follower
     tokens; over calibration inputs the scores are averaged (fp64, input order)
     and the head is marked when the average is strictly above gamma;
  R22 a later search reuses the LSE cached by an earlier one as it is (no
     correction): each row's energy terms are then scaled by one factor per row;
  R25 heavy rows (more kept blocks than a factor times the mean) run first.

Parity pins: every function is pinned by tests against library routines, closed
forms, invariants or brute force (tests/test_oracle.py).
"""
import math

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _scale(d, scale):
    return 1.0 / math.sqrt(d) if scale is None or scale == 0 else float(scale)


def _softmax_rows(s):
    """Exact row softmax of logits s [r, n] in fp64 with its log-sum-exp."""
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    return e / l, (m + np.log(l))[:, 0]


def dense_attention(q, k, v, scale=None):
    """softmax(Q K^T * scale) V over all N keys, with LSE_i = log sum_j exp(s_ij).

    The quadratic dense attention that the CalibAtt summaries name as the cost
    being cut ([CA-zh] S1; [CA-de] S1) and that the speedups are measured against.
    Returns (o [N, d], lse [N]) in fp64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    c = _scale(q.shape[1], scale)
    s = (q @ k.T) * c
    p, lse = _softmax_rows(s)
    return p @ v, lse


def block_energy(q, k, block, scale=None, q_blocks=None):
    """Block energy E[qb, kb] = sum_{i in qb} sum_{j in kb} P_ij, P = softmax over
    all keys of the dense attention.

    [CA-zh] S2.2A and [CA-fr] S2B.1: the attention matrix of a calibration input is
    cut into B x B tiles and each query block's energy towards each key block is the
    sum of the attention scores in the tile (R1: raw sum, so a ragged block simply
    holds less energy).  Returns fp64 [nqb, nkb], or only the rows listed in
    q_blocks.
    """
    q, k = _f64(q), _f64(k)
    n = q.shape[0]
    c = _scale(q.shape[1], scale)
    nb = (n + block - 1) // block
    starts = np.arange(0, n, block)
    rows = range(nb) if q_blocks is None else q_blocks
    out = np.zeros((len(rows), nb), dtype=np.float64)
    for r, qb in enumerate(rows):
        lo, hi = qb * block, min(n, (qb + 1) * block)
        p, _ = _softmax_rows((q[lo:hi] @ k.T) * c)
        col = p.sum(axis=0)  # sum over the query rows of the tile
        out[r] = np.add.reduceat(col, starts)  # then over the key tokens of each block
    return out


def block_energy_from_lse(q, k, lse, block, scale=None, q_blocks=None):
    """Block energy from a given log-sum-exp: E[qb, kb] = sum over i in qb and j in kb
    of exp(s_ij - lse_i).

    [AdaSpa] S2: the search pass caches the LSE of the dense attention it computes,
    and later searches reuse that cache instead of recomputing it; [CA-zh] S2.2A for
    the tile energy.  With the LSE of the same q and k this is block_energy; with an
    LSE cached from another input (an earlier denoising step) each row's terms are
    that row's probabilities times exp(lse_true_i - lse_i) (R22).  lse: [N], natural
    log.  Returns fp64 [nqb, nkb], or the rows listed in q_blocks.
    """
    q, k, lse = _f64(q), _f64(k), _f64(lse)
    n = q.shape[0]
    c = _scale(q.shape[1], scale)
    nb = (n + block - 1) // block
    starts = np.arange(0, n, block)
    rows = range(nb) if q_blocks is None else q_blocks
    out = np.zeros((len(rows), nb), dtype=np.float64)
    for r, qb in enumerate(rows):
        lo, hi = qb * block, min(n, (qb + 1) * block)
        w = np.exp((q[lo:hi] @ k.T) * c - lse[lo:hi, None])
        out[r] = np.add.reduceat(w.sum(axis=0), starts)
    return out


def select_row(e, tau):
    """Fewest key blocks, highest energy first, whose cumulative energy reaches
    tau times the row total.

    [CA-zh] S2.2A (keep the highest-energy key blocks for each query block under the
    threshold), [CA-de] S2A.2 (blocks carrying a given share of the total energy),
    [CA-fr] S2B.1 (minimal number of key blocks reaching the cumulative threshold).
      order : key blocks by (energy descending, index ascending)        (R4)
      S_k   : fp64 running sum, added one term at a time in that order
      T     : S over all blocks (the row total)                          (R2)
      keep  : the first k* blocks, k* = min{k >= 1 : S_k >= tau * T}     (R3)
    tau >= 1 keeps all blocks (R5).  Returns bool [nkb].
    """
    e = _f64(e)
    nkb = e.shape[0]
    keep = np.zeros(nkb, dtype=bool)
    if tau >= 1.0:
        keep[:] = True
        return keep
    order = np.lexsort((np.arange(nkb), -e))
    running = np.cumsum(e[order])  # sequential: running[i] = running[i-1] + e[order[i]]
    target = tau * running[-1]
    kstar = int(np.argmax(running >= target)) + 1
    keep[order[:kstar]] = True
    return keep


def aggregate_votes(votes, n_draws, rho):
    """Keep a block when the fraction of calibration inputs that kept it is above rho.

    [CA-zh] S2.2A cross-prompt aggregation (average the binary masks into a keep
    frequency; keep above the agreement threshold rho, e.g. 0.5); [CA-fr] S2B.2.
    R6: strict comparison of the integer vote count with rho * n_draws in fp64.
    """
    return np.asarray(votes) > (float(rho) * float(n_draws))


def select_blocks(energy, tau, rho=0.5, force_diag=True, n_dense_prefix_blocks=0):
    """Calibrated mask from per-draw block energies.

    energy: [draws, heads, nqb, nkb]. Per draw and row: select_row; then votes over
    draws and aggregate_votes; then R7 forcing (diagonal; rows and columns of the
    first n_dense_prefix_blocks blocks).  tau is one threshold, or one per head (the
    per-head recall targets of [AdaSpa] S2, head-adaptive sparsity).  Returns
    (mask uint8 [heads, nqb, nkb], votes int32 [heads, nqb, nkb]).
    """
    energy = _f64(energy)
    n_draws, heads, nqb, nkb = energy.shape
    taus = np.broadcast_to(np.asarray(tau, dtype=np.float64), (heads,))
    votes = np.zeros((heads, nqb, nkb), dtype=np.int32)
    for d in range(n_draws):
        for h in range(heads):
            for qb in range(nqb):
                votes[h, qb] += select_row(energy[d, h, qb], taus[h])
    mask = aggregate_votes(votes, n_draws, rho)
    if force_diag:
        idx = np.arange(min(nqb, nkb))
        mask[:, idx, idx] = True
    if n_dense_prefix_blocks > 0:
        p = int(n_dense_prefix_blocks)
        mask[:, :p, :] = True
        mask[:, :, :p] = True
    return mask.astype(np.uint8), votes


def build_csr(mask):
    """Mask rows -> lists of kept key-block indices (the summaries' skip lists).

    [CA-zh] S2.2B (the mask becomes a list of the block intervals to compute),
    [CA-pt] S2A.5, [CA-fr] S2C.  Layout: row_ptr[0] = 0,
    row_ptr[r+1] = row_ptr[r] + (kept blocks in row r); col_idx holds each row's
    kept indices in ascending order; work_order lists the rows by kept count
    descending, ties by ascending row (the longest-first order used to balance
    heads of differing density, [AdaSpa] S2).  mask: [rows, nkb].
    """
    mask = np.asarray(mask).astype(bool)
    rows = mask.shape[0]
    counts = mask.sum(axis=1).astype(np.int64)
    row_ptr = np.zeros(rows + 1, dtype=np.int32)
    row_ptr[1:] = np.cumsum(counts)
    col_idx = np.nonzero(mask)[1].astype(np.int32)  # row-major scan: ascending per row
    work_order = np.argsort(-counts, kind="stable").astype(np.int32)
    return row_ptr, col_idx, work_order


def heavy_first_order(counts, factor):
    """Processing order of skip-list rows: the heavy rows first, the rest in place.

    [AdaSpa] S2 balances the work of rows (heads) of differing density; here only
    the rows much longer than the average are moved ahead, so that no long row
    starts last, while the others keep the natural order that neighbouring rows
    share keys in (R25).  heavy: kept count > factor * (mean kept count), compared
    in fp64; heavy rows by (count descending, row ascending), then the other rows
    ascending.  counts: [rows].  Returns int32 [rows].
    """
    counts = np.asarray(counts, dtype=np.int64)
    thr = float(factor) * (float(counts.sum()) / float(counts.size))
    heavy = np.nonzero(counts > thr)[0]
    heavy = heavy[np.argsort(-counts[heavy], kind="stable")]
    light = np.nonzero(counts <= thr)[0]
    return np.concatenate([heavy, light]).astype(np.int32)


def build_intervals(mask):
    """Mask rows -> runs of consecutive kept key blocks, the summaries' "block
    intervals" of the skip list.

    [CA-zh] S2.2B: the mask is turned into a skip list holding only the block
    intervals to compute.  Layout: iv_ptr[0] = 0, iv_ptr[r+1] = iv_ptr[r] + (runs of
    row r); run j of the row starts at key block first[j] and covers count[j] >= 1
    consecutive kept blocks; a row's runs are ascending and maximal (a skipped block
    separates any two).  work_order is that of build_csr (kept blocks descending,
    ties by ascending row).  mask: [rows, nkb].  Returns (iv_ptr, first, count,
    work_order).
    """
    mask = np.asarray(mask).astype(bool)
    rows, nkb = mask.shape
    edge = np.zeros((rows, nkb + 1), dtype=np.int8)
    edge[:, :nkb] += mask
    edge[:, 1:] -= mask  # +1 where a run starts, -1 just past where one ends
    r_start, c_start = np.nonzero(edge == 1)
    _, c_end = np.nonzero(edge == -1)  # row-major scans: the ends pair with the starts in order
    iv_ptr = np.zeros(rows + 1, dtype=np.int32)
    iv_ptr[1:] = np.cumsum(np.bincount(r_start, minlength=rows))
    _, _, work_order = build_csr(mask)
    return iv_ptr, c_start.astype(np.int32), (c_end - c_start).astype(np.int32), work_order


def computed_rows(seq_len, n_prefix, grid, anchor_stride, is_rep_head):
    """Query rows that attention computes: all rows for a normal head; for a spatial
    repetition head the text rows and the anchor rows (R8).

    [CA-zh] S2.1 and S2.2B, [CA-fr] S2A.4 and S2C: for heads marked repeating only
    a few anchor rows of each frame are computed.
    """
    rows = np.ones(seq_len, dtype=bool)
    if not is_rep_head:
        return rows
    f_, h_, w_ = grid
    t = np.arange(n_prefix, seq_len)
    y = ((t - n_prefix) // w_) % h_
    rows[n_prefix:] = (y % anchor_stride) == 0
    return rows


def token_mask_from_blocks(mask_h, block, n):
    """Expand a [nqb, nkb] block mask to the [N, N] token mask it stands for."""
    mask_h = np.asarray(mask_h).astype(bool)
    blk = np.arange(n) // block
    return mask_h[np.ix_(blk, blk)]


def sparse_attention(q, k, v, mask_h, block, scale=None, rows=None):
    """Exact attention restricted to the kept key blocks of each query block.

    [CA-zh] S2.2B and [CA-de] S2B: only the selected blocks are computed (densely)
    and the others are skipped; a skipped block takes no part in the softmax.
    For query row i in block qb(i): o_i = sum_j softmax_j(s_ij) v_j with j over the
    tokens of the key blocks kept in mask row qb(i).  `rows` (bool [N] or index
    list) limits the rows computed; rows not computed get o = 0 and lse = -inf, and
    so does a row whose mask row keeps nothing.  Returns (o [N, d], lse [N]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    n, d = q.shape
    c = _scale(d, scale)
    mask_h = np.asarray(mask_h).astype(bool)
    if rows is None:
        want = np.ones(n, dtype=bool)
    else:
        rows = np.asarray(rows)
        if rows.dtype == bool:
            want = rows
        else:
            want = np.zeros(n, dtype=bool)
            want[rows] = True
    o = np.zeros((n, v.shape[1]), dtype=np.float64)
    lse = np.full(n, -np.inf, dtype=np.float64)
    nqb = (n + block - 1) // block
    for qb in range(nqb):
        qi = np.nonzero(want[qb * block:(qb + 1) * block])[0] + qb * block
        if qi.size == 0:
            continue
        kept = np.nonzero(mask_h[qb])[0]
        if kept.size == 0:
            continue
        kj = np.concatenate([np.arange(kb * block, min(n, (kb + 1) * block)) for kb in kept])
        p, l = _softmax_rows((q[qi] @ k[kj].T) * c)
        o[qi] = p @ v[kj]
        lse[qi] = l
    return o, lse


def row_broadcast(o, n_prefix, grid, anchor_stride):
    """Copy each anchor row's output to the rows it stands for in the same frame.

    [CA-zh] S2.1 (compute a few anchor rows and broadcast them to the other rows of
    the frame), [CA-fr] S2C.  O[f, y, x] <- O[f, s*floor(y/s), x] for grid tokens;
    text tokens are untouched (R8, R9).  Returns a new array.
    """
    out = np.array(o, copy=True)
    f_, h_, w_ = grid
    s = int(anchor_stride)
    if s <= 1:
        return out
    g = out[n_prefix:n_prefix + f_ * h_ * w_].reshape(f_, h_, w_, -1)
    anchors = (np.arange(h_) // s) * s
    out[n_prefix:n_prefix + f_ * h_ * w_] = g[:, anchors].reshape(f_ * h_ * w_, -1)
    return out


def sparse_attention_with_repetition(q, k, v, mask_h, block, n_prefix, grid, anchor_stride,
                                     is_rep_head, scale=None):
    """One head of the inference path: block-sparse attention on the computed rows,
    then, for a repetition head, the anchor broadcast.  Block sparsity and row
    repetition apply together ([CA-zh] S3: the two strategies are complementary).
    The follower rows' LSE is the anchor's.  Returns (o, lse)."""
    n = q.shape[0]
    rows = computed_rows(n, n_prefix, grid, anchor_stride, is_rep_head)
    o, lse = sparse_attention(q, k, v, mask_h, block, scale, rows)
    if is_rep_head:
        o = row_broadcast(o, n_prefix, grid, anchor_stride)
        lse = row_broadcast(lse[:, None], n_prefix, grid, anchor_stride)[:, 0]
    return o, lse


def _follower_anchor_pairs(seq_len, n_prefix, grid, anchor_stride):
    """Follower grid tokens (y mod s != 0, ascending) and the anchor token of each,
    (f, s*floor(y/s), x) in the same frame and column (R8, R9)."""
    f_, h_, w_ = grid
    s = int(anchor_stride)
    t = np.arange(n_prefix, seq_len)
    y = ((t - n_prefix) // w_) % h_
    follower = t[y % s != 0]
    anchor = follower - (y[y % s != 0] % s) * w_
    return follower, anchor


def repetition_cosines(q, k, n_prefix, grid, anchor_stride, scale=None, tokens=None):
    """Cosine similarity between the attention vector of each follower token and
    that of its anchor, for one head.

    [CA-zh] S2.2A (spatial repetition detection: the cosine similarity of attention
    vectors between different spatial rows of one frame) and [CA-fr] S2B.3 (the same
    between the spatial rows of one image).  R17: the attention vector of token i is
    P_i = softmax_j(s_ij) over all N keys; follower i is paired with its anchor a(i),
    the token whose output the broadcast copies into i, and
        cos_i = <P_i, P_a(i)> / (|P_i| |P_a(i)|).
    tokens: optional follower tokens to evaluate (default: every follower).  Needs
    anchor_stride >= 2 and at least one follower.  Returns (tokens, cos) in fp64.
    """
    q, k = _f64(q), _f64(k)
    n = q.shape[0]
    c = _scale(q.shape[1], scale)
    follower, anchor = _follower_anchor_pairs(n, n_prefix, grid, anchor_stride)
    if int(anchor_stride) < 2 or follower.size == 0:
        raise ValueError("repetition detection needs anchor_stride >= 2 and follower rows")
    if tokens is not None:
        tokens = np.asarray(tokens, dtype=np.int64)
        pos = np.searchsorted(follower, tokens)
        if np.any(pos >= follower.size) or np.any(follower[np.minimum(pos, follower.size - 1)] != tokens):
            raise ValueError("tokens must be follower tokens")
        follower, anchor = follower[pos], anchor[pos]
    p_f, _ = _softmax_rows((q[follower] @ k.T) * c)
    p_a, _ = _softmax_rows((q[anchor] @ k.T) * c)
    cos = (p_f * p_a).sum(axis=1) / (np.sqrt((p_f * p_f).sum(axis=1)) * np.sqrt((p_a * p_a).sum(axis=1)))
    return follower, cos


def repetition_score(q, k, n_prefix, grid, anchor_stride, scale=None):
    """Repetition score of one head: the mean of repetition_cosines over all its
    follower tokens (R18).  Returns (score, cos [N] with NaN at non-followers)."""
    n = q.shape[0]
    tokens, cos = repetition_cosines(q, k, n_prefix, grid, anchor_stride, scale)
    full = np.full(n, np.nan)
    full[tokens] = cos
    return float(cos.mean()), full


def mark_repetition_heads(scores, gamma):
    """Repetition flags from per-input head scores.

    [CA-zh] S2.2A: a (timestep, layer, head) whose similarity exceeds gamma is marked
    spatially repetitive; [CA-fr] S2B.3: the head is marked repetitive.  R18: scores
    is [n_draws, heads]; each head's scores are added one at a time in fp64 in draw
    order, divided by n_draws, and compared strictly with gamma.  Returns uint8
    [heads].
    """
    scores = np.asarray(scores)
    n_draws, heads = scores.shape
    out = np.zeros(heads, dtype=np.uint8)
    for h in range(heads):
        acc = 0.0
        for d in range(n_draws):
            acc += float(scores[d, h])
        out[h] = 1 if acc / n_draws > float(gamma) else 0
    return out
