/*
 * calibattn.h -- C ABI of libcalibattn.so: calibrated block-sparse spatiotemporal
 * self-attention for video diffusion transformers on AMD MI355X (gfx950).
 *
 * The method (CalibAtt, "Accelerating Text-to-Video Generation with Calibrated
 * Sparse Attention"; technical summaries on gist.science in zh/de/pt/fr) has an
 * offline calibration stage and an inference stage:
 *   calibration (zh S2.2A, de S2A, fr S2B): per calibration input, the attention
 *     matrix is cut into B x B tiles, each tile's energy is the sum of its attention
 *     probabilities, each query block keeps the fewest highest-energy key blocks that
 *     reach a threshold, and the per-input masks are aggregated by vote; heads whose
 *     attention rows repeat across the image rows of a frame are marked for
 *     anchor-row computation;
 *   inference (zh S2.2B, de S2B, fr S2C): the mask becomes a skip list and a kernel
 *     computes attention over the kept blocks only; for heads marked spatially
 *     repetitive only anchor rows are computed and then broadcast in their frame.
 * The energy pass caches the log-sum-exp of a dense pass and reuses it, and work
 * is balanced across heads of differing density, as in AdaSpa ("Training-free and
 * Adaptive Sparse Attention for Efficient Long Video Generation", S2 method).
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked (host).  The caller allocates and
 *     frees every buffer; the library allocates nothing and keeps no state, so the
 *     calls are thread-safe.  The one exception is calib_block_energy_noalloc,
 *     whose fixed per-GPU array is shared by its calls on that GPU (see there).
 *   - Each call validates its arguments on the host and either returns an error
 *     without enqueuing anything, or enqueues its kernels on `stream` and returns
 *     at once (no synchronisation).  Faults inside kernels surface at the
 *     caller's next synchronisation.
 *   - Q, K, V, O are [batch, heads, seq_len, head_dim] with the element strides in
 *     the descriptor and head_dim contiguous.  Tokens are in frame-major order:
 *     n_prefix non-grid (text) tokens first, then token
 *     n_prefix + f*grid_h*grid_w + y*grid_w + x for grid position (f, y, x).
 *   - Blocks are contiguous runs of `block` tokens; nb = ceil(seq_len / block) and
 *     the last block may be ragged.  A block mask is uint8 [heads, nb, nb] with
 *     1 = kept, shared by every batch item.
 *   - LSE is fp32 [batch, heads, seq_len], natural log.
 *   - The default softmax scale (scale == 0) is 1/sqrt(head_dim).
 */
#ifndef CALIBATTN_H
#define CALIBATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* cba_stream_t; /* a hipStream_t; NULL = the null stream */

typedef int32_t cba_status;
#define CBA_OK 0
#define CBA_EINVAL 1       /* bad shape, stride, pointer, alignment or parameter */
#define CBA_EUNSUPPORTED 2 /* unsupported dtype / head_dim / block combination */
#define CBA_EHIP 3         /* a HIP launch failed; nothing after it was enqueued */
#define CBA_ECAPACITY 4    /* a caller buffer is too small for the request */

#define CBA_DTYPE_F32 0
#define CBA_DTYPE_BF16 1

/* Shape and layout of one attention problem.  batch, heads and seq_len are at
 * least 1 (an empty problem is CBA_EINVAL, not a no-op).  head_dim is 64 or 128;
 * block is 32, 64 or 128.  n_prefix must be a multiple of block.  grid_f*grid_h*grid_w is
 * either 0 (no token grid: repetition heads are then not allowed) or
 * seq_len - n_prefix.  bf16 needs 16-byte aligned tensor pointers and strides
 * that are multiples of 8 elements. */
typedef struct cba_attn_desc {
  int32_t dtype;
  int32_t batch, heads, seq_len, head_dim;
  int32_t block;
  int32_t n_prefix;
  int32_t grid_f, grid_h, grid_w;
  float scale;
  int64_t stride_b, stride_h, stride_n; /* element strides shared by Q, K, V, O */
} cba_attn_desc;

/* Block energy of dense attention, with the log-sum-exp cached between sweeps.
 * (zh S2.2A, fr S2B.1: E[qb,kb] is the sum of the attention probabilities of
 * the tile; AdaSpa S2: the dense pass caches its LSE and the search reuses it.)
 *   sweep 1: a dense attention pass writes lse (and o when v and o are given);
 *   sweep 2: recomputes the scores, adds exp(s_ij - lse_i) over each tile, writes
 *            energy[b, h, qb, kb] (fp32, contiguous [batch, heads, nb, nb]).
 * The batch index is the calibration input (draw).  v and o are both NULL or both
 * set.  Every energy entry is written; each is the sum of one tile in a fixed
 * order, so repeated calls give identical bits. */
cba_status calib_block_energy(const cba_attn_desc* desc, const void* q, const void* k,
                              const void* v, void* o, float* lse, float* energy,
                              cba_stream_t stream);

/* calib_block_energy in a single pass over the keys (bf16), with a caller
 * workspace instead of the second sweep.  For each row and key block the pass
 * stores the block's base-2 log-sum of the scaled scores in the workspace; once
 * the row's log-sum-exp is known the workgroup adds exp(.. - lse_i) of its rows per
 * block (zh S2.2A: E[qb, kb] = sum of the tile's attention probabilities).
 * Arguments and outputs as calib_block_energy: v and o both NULL or both set; with
 * V the pass also writes O.  lse and O are bit-identical to calib_block_energy's
 * (and dense_attn_fwd's); each energy entry is the sum of one tile in a fixed
 * order (repeated calls give identical bits; they may differ from
 * calib_block_energy's by rounding).
 *   workspace: device, 16-byte aligned, workspace_bytes long; its contents on
 *              entry do not matter and are left undefined.  With batch * heads *
 *              nb * nb * block floats the pass runs in one launch; a smaller
 *              workspace runs it in several launches over contiguous (batch item,
 *              head, query block) ranges, each holding its rows' log-sums, with
 *              bit-identical results.  CBA_ECAPACITY (nothing enqueued) when it
 *              cannot hold one workgroup's rows (up to 8 query blocks x nb x block
 *              floats).
 * fp32 inputs run the two sweeps and do not use the workspace. */
cba_status calib_block_energy_ws(const cba_attn_desc* desc, const void* q, const void* k, const void* v, void* o,
                                 float* lse, float* energy, void* workspace, int64_t workspace_bytes,
                                 cba_stream_t stream);

/* calib_block_energy_ws for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * no workspace argument.  The log-sums go to a fixed 256 MiB device array of the
 * library, one per GPU, held from the first call on that GPU until the process
 * ends; the call allocates nothing.  When the problem's workspace
 * (batch * heads * nb * nb * block floats) exceeds the array, the work runs in
 * several consecutive launches over contiguous (batch item, head, query block)
 * ranges; results are bit-identical to calib_block_energy_ws's.  CBA_ECAPACITY
 * (nothing enqueued) only if one workgroup's rows alone exceed the array.
 * Calls that overlap in time on one GPU (two streams or threads) share the array
 * and race: the caller must serialise them.  The stream must belong to the
 * current device (CBA_EINVAL otherwise).  Arguments, outputs and the fp32 case
 * as calib_block_energy_ws. */
cba_status calib_block_energy_noalloc(const cba_attn_desc* desc, const void* q, const void* k, const void* v,
                                      void* o, float* lse, float* energy, cba_stream_t stream);

/* Block energy sweep alone, from a given log-sum-exp ([AdaSpa] S2: the search pass
 * caches the LSE of its dense pass and later searches reuse that cache; zh S2.2A
 * for the tile energy).  energy[b, h, qb, kb] = sum over i in qb and j in kb of
 * exp(s_ij - lse[b, h, i]).  With the LSE of the same q and k (calib_block_energy,
 * dense_attn_fwd) this is calib_block_energy's sweep 2, bit for bit; with an LSE
 * cached from an earlier input each row's terms carry one factor per row.
 *   lse: fp32 [batch, heads, seq_len], natural log (read only).
 *   energy: fp32 [batch, heads, nb, nb] output; every entry written, each the sum of
 *           one tile in a fixed order. */
cba_status block_energy_from_lse(const cba_attn_desc* desc, const void* q, const void* k, const float* lse,
                                 float* energy, cba_stream_t stream);

/* Calibrated block mask from per-draw energies (zh S2.2A; de S2A.2-3; fr S2B.1-2).
 *   energy: fp32 [n_draws, heads, nb, nb] (as written by calib_block_energy).
 *   Per draw and row, key blocks are ordered by (energy descending, index
 *   ascending); the running sum S_k is accumulated in fp64 one term at a time in
 *   that order; T is the full sum; the first k* blocks are kept, with
 *   k* = min{k >= 1 : S_k >= tau * T}.  tau >= 1 keeps every block.
 *   A block is kept in the result when its vote count over the draws is strictly
 *   greater than rho * n_draws (fp64).  Then, when force_diag != 0, the diagonal
 *   block of every row is set, and the rows and columns of the first
 *   n_dense_prefix_blocks blocks are set.
 *   mask: uint8 [heads, nb, nb] (output).  votes: optional int32 [heads, nb, nb].
 * nb <= 4096.  Results are bit-exact functions of the energy bits. */
cba_status select_blocks_by_energy(const float* energy, int32_t n_draws, int32_t heads, int32_t nb,
                                   double tau, double rho, int32_t force_diag,
                                   int32_t n_dense_prefix_blocks, uint8_t* mask, int32_t* votes,
                                   cba_stream_t stream);

/* select_blocks_by_energy with one energy threshold per head (the per-head recall
 * targets of head-adaptive sparsity, [AdaSpa] S2): row (h, qb) keeps the fewest
 * blocks reaching tau_heads[h] of its energy; everything else as in
 * select_blocks_by_energy.  tau_heads (host): double [heads], each finite and
 * >= 0; heads <= 256. */
cba_status select_blocks_by_energy_heads(const float* energy, int32_t n_draws, int32_t heads, int32_t nb,
                                         const double* tau_heads, double rho, int32_t force_diag,
                                         int32_t n_dense_prefix_blocks, uint8_t* mask, int32_t* votes,
                                         cba_stream_t stream);

/* Skip list of a block mask in CSR form (zh S2.2B; pt S2A.5; fr S2C).
 *   mask: uint8 [n_rows, nkb] (1 = kept); for attention, n_rows = heads * nb and
 *         row r = h * nb + qb.  n_rows and nkb are at least 1 (CBA_EINVAL).
 *   row_ptr: int32 [n_rows + 1], row_ptr[0] = 0, row_ptr[r+1] - row_ptr[r] = kept
 *            blocks of row r.  Always written.
 *   col_idx: int32 [col_idx_capacity] or NULL.  NULL = count pass only.  Otherwise
 *            each row's kept block indices in ascending order at
 *            [row_ptr[r], row_ptr[r+1]); entries at or beyond col_idx_capacity are
 *            not written (row_ptr[n_rows] > col_idx_capacity tells the caller).  A
 *            capacity of n_rows * nkb can never be exceeded.
 *   work_order: int32 [n_rows] or NULL: the rows sorted by kept count descending,
 *            ties by ascending row index (longest-first order for load balance
 *            across heads of differing density, AdaSpa S2).
 * Integer results, bit-exact. */
cba_status build_block_csr(const uint8_t* mask, int32_t n_rows, int32_t nkb, int32_t* row_ptr,
                           int32_t* col_idx, int64_t col_idx_capacity, int32_t* work_order,
                           cba_stream_t stream);

/* Processing order of skip-list rows with only the heavy rows moved ahead (AdaSpa
 * S2 balances the work of rows of differing density).  A row is heavy when its
 * kept count row_ptr[r+1] - row_ptr[r] is above factor * (row_ptr[n_rows] /
 * n_rows), computed in fp64.  work_order lists the heavy rows by (count
 * descending, row ascending), then every other row in ascending order: long rows
 * (such as the dense rows of text tokens) no longer start last, while the others
 * keep the natural order in which neighbouring rows share key blocks.  factor = 0
 * gives build_block_csr's longest-first order; a factor no row reaches gives the
 * natural order.
 *   row_ptr: int32 [n_rows + 1] from build_block_csr for a mask of nkb columns
 *            (every count in [0, nkb]).
 *   work_order: int32 [n_rows] output, a permutation of the rows.
 * factor finite and >= 0.  Integer results, bit-exact. */
cba_status order_heavy_rows_first(const int32_t* row_ptr, int32_t n_rows, int32_t nkb, double factor,
                                  int32_t* work_order, cba_stream_t stream);

/* Skip list as block intervals (zh S2.2B: the mask becomes a skip list holding
 * only the block intervals to compute): the maximal runs of consecutive kept
 * blocks of each mask row.  A compact form of the skip list for the per
 * (timestep, layer, head) mask dictionary: a banded mask row is a few runs where
 * its CSR row holds every block.
 *   mask: uint8 [n_rows, nkb] (1 = kept), nkb <= 65535.
 *   iv_ptr: int32 [n_rows + 1], iv_ptr[0] = 0, iv_ptr[r+1] - iv_ptr[r] = runs of
 *           row r.  Always written.
 *   ivs: uint32 [iv_capacity] or NULL (count pass only).  Run j of row r is
 *           ivs[iv_ptr[r] + j] = first | (count << 16): blocks first .. first +
 *           count - 1 are kept, count >= 1; a row's runs are ascending and a
 *           skipped block separates any two.  Entries at or beyond iv_capacity are
 *           not written (iv_ptr[n_rows] > iv_capacity tells the caller); a capacity
 *           of n_rows * ceil(nkb / 2) can never be exceeded.
 * For the longest-first row order, call build_block_csr with col_idx = NULL.
 * Integer results, bit-exact. */
cba_status build_block_intervals(const uint8_t* mask, int32_t n_rows, int32_t nkb, int32_t* iv_ptr,
                                 uint32_t* ivs, int64_t iv_capacity, cba_stream_t stream);

/* Exact attention over the kept key blocks only (zh S2.2B; de S2B; fr S2C).
 * For query token i in query block qb of head h, o_i = sum_j softmax_j(s_ij) v_j
 * with s_ij = scale * q_i . k_j and j over the tokens of the key blocks listed for
 * row r = h * nb + qb in col_idx[row_ptr[r] .. row_ptr[r+1]); unlisted blocks take
 * no part in the softmax.  A row with no listed block gives o = 0, lse = -inf.
 *   row_ptr/col_idx: as written by build_block_csr for a [heads, nb, nb] mask;
 *            col_idx_len = number of valid col_idx entries (entries outside
 *            [0, nb) and positions at or beyond col_idx_len are ignored).
 *   work_order: optional int32 [heads * nb] processing order of the rows (as from
 *            build_block_csr); NULL = ascending rows.  Entries outside
 *            [0, heads * nb) are skipped.
 *   rep_heads (host): optional uint8 [heads]; a nonzero entry marks a spatial
 *            repetition head (zh S2.1, S2.2B; fr S2A.4, S2C): only its text tokens
 *            and the grid tokens with y % anchor_stride == 0 (anchor rows) are
 *            computed, each with its own query block's mask.  Their lse is also
 *            written to the follower rows (y % anchor_stride != 0) of the anchor's
 *            group.  With fuse_broadcast != 0 the anchor outputs are written to the
 *            followers too; otherwise call rep_row_broadcast afterwards.
 *            heads <= 1024 when rep_heads is given; anchor_stride >= 1.
 *   o: output; lse: optional output. */
cba_status sparse_attn_fwd(const cba_attn_desc* desc, const void* q, const void* k, const void* v,
                           const int32_t* row_ptr, const int32_t* col_idx, int64_t col_idx_len,
                           const int32_t* work_order, const uint8_t* rep_heads,
                           int32_t anchor_stride, int32_t fuse_broadcast, void* o, float* lse,
                           cba_stream_t stream);

/* sparse_attn_fwd with the skip list given as block intervals (zh S2.2B), as
 * written by build_block_intervals for a [heads, nb, nb] mask: row r = h * nb + qb
 * visits the blocks of runs ivs[iv_ptr[r] .. iv_ptr[r+1]) in order.  iv_len =
 * number of valid ivs entries (positions at or beyond it are ignored; blocks
 * outside [0, nb) are skipped).  Every other argument and every result as in
 * sparse_attn_fwd; the same mask gives bit-identical outputs through either
 * call. */
cba_status sparse_attn_fwd_intervals(const cba_attn_desc* desc, const void* q, const void* k, const void* v,
                                     const int32_t* iv_ptr, const uint32_t* ivs, int64_t iv_len,
                                     const int32_t* work_order, const uint8_t* rep_heads, int32_t anchor_stride,
                                     int32_t fuse_broadcast, void* o, float* lse, cba_stream_t stream);

/* Anchor-row broadcast for spatial repetition heads (zh S2.1; fr S2C):
 * O[b, h, f, y, x] <- O[b, h, f, anchor_stride * floor(y / anchor_stride), x] for
 * every grid token of every head with rep_heads[h] != 0.  Text tokens are not
 * touched.  A plain copy: bit-exact.  rep_heads (host) uint8 [heads], heads <= 1024. */
cba_status rep_row_broadcast(const cba_attn_desc* desc, void* o, const uint8_t* rep_heads,
                             int32_t anchor_stride, cba_stream_t stream);

/* Dense attention softmax(Q K^T * scale) V over all keys: the baseline the sparse
 * path is measured against (zh S1; pt S4).  Same kernels as sparse_attn_fwd with
 * every key block listed.  lse optional. */
cba_status dense_attn_fwd(const cba_attn_desc* desc, const void* q, const void* k, const void* v,
                          void* o, float* lse, cba_stream_t stream);

/* Spatial-repetition similarity of every head, from one dense pass per
 * calibration input (zh S2.2A, spatial repetition detection: cosine similarity of
 * the attention vectors of different spatial rows of one frame; fr S2B.3).
 * The attention vector of token i is its row of dense attention probabilities,
 * P_i[j] = exp(s_ij - lse_i) over all seq_len keys.  Each follower grid token
 * i = (f, y, x), y % anchor_stride != 0, is compared with its anchor
 * a(i) = (f, anchor_stride * floor(y / anchor_stride), x), the token whose output
 * rep_row_broadcast copies into it:
 *     token_cos[b, h, i] = <P_i, P_a(i)> / (|P_i| |P_a(i)|),
 * and head_sim[b, h] is the mean of token_cos over the follower tokens of (b, h).
 *   lse: fp32 [batch, heads, seq_len], natural log, as written for the same q and k
 *        by calib_block_energy or dense_attn_fwd.  It only sets the scale of each
 *        row's exponentials: the cosine does not depend on it beyond rounding.
 *   token_cos: fp32 [batch, heads, seq_len] output, written at follower tokens
 *        only; every other entry is left as it was.
 *   head_sim: fp32 [batch, heads] output.  Each is a sum in a fixed order, so
 *        repeated calls give identical bits.
 * The batch index is the calibration input.  Needs a token grid, grid_h >= 2 and
 * anchor_stride >= 2 (so that follower rows exist); desc->block is not used and
 * n_prefix need not be a multiple of it.
 * q and k as for calib_block_energy. */
cba_status spatial_rep_similarity(const cba_attn_desc* desc, const void* q, const void* k, const float* lse,
                                  int32_t anchor_stride, float* token_cos, float* head_sim,
                                  cba_stream_t stream);

/* Repetition flags from the per-input head similarities (zh S2.2A: a (timestep,
 * layer, head) whose similarity exceeds gamma is marked spatially repetitive;
 * fr S2B.3).  rep_heads[h] = 1 when the mean over the n_draws rows of
 * head_sim[:, h], added in fp64 one draw at a time in draw order and divided by
 * n_draws, is strictly greater than gamma; else 0.
 *   head_sim: fp32 [n_draws, heads] (spatial_rep_similarity with batch = n_draws).
 *   rep_heads: uint8 [heads] device output (copy it to the host for
 *        sparse_attn_fwd and rep_row_broadcast).
 * A bit-exact function of the head_sim bits. */
cba_status select_rep_heads(const float* head_sim, int32_t n_draws, int32_t heads, double gamma,
                            uint8_t* rep_heads, cba_stream_t stream);

/* Static description of a status code. */
const char* cba_status_str(cba_status status);

/* Library version, e.g. 100 for 0.1.0. */
int32_t cba_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CALIBATTN_H */
