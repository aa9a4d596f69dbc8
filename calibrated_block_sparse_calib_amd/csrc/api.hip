// C ABI of libcalibattn.so: argument validation on the host and dispatch to the
// kernels.  Every entry point either returns an error before enqueuing anything or
// enqueues its kernels on the caller's stream and returns without waiting.
#include "api_checks.h"

using namespace cba::abi;
using cba::AttnParams;

CBA_API cba_status calib_block_energy(const cba_attn_desc* desc, const void* q, const void* k, const void* v,
                                      void* o, float* lse, float* energy, cba_stream_t stream) {
  cba_status st = check_desc(desc);
  if (st) return st;
  if (check_tensor(q) || check_tensor(k) || !lse || !energy) return CBA_EINVAL;
  if ((v == nullptr) != (o == nullptr)) return CBA_EINVAL;
  if (v && (check_tensor(v) || check_tensor(o))) return CBA_EINVAL;
  AttnParams p = make_params(desc);
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.energy = energy;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // Sweep 1: dense pass, caches LSE (and writes O when V is given).
  hipError_t e = run_attention(p, desc, /*with_pv=*/v != nullptr, s);
  if (e != hipSuccess) return from_hip(e);
  // Sweep 2: tile sums of exp(s - lse).
  e = desc->dtype == CBA_DTYPE_BF16 ? cba::launch_energy_bf16(p, desc->head_dim, desc->block, s)
                                    : cba::launch_energy_f32(p, desc->head_dim, desc->block, s);
  return from_hip(e);
}

CBA_API cba_status calib_block_energy_ws(const cba_attn_desc* desc, const void* q, const void* k, const void* v,
                                         void* o, float* lse, float* energy, void* workspace,
                                         int64_t workspace_bytes, cba_stream_t stream) {
  cba_status st = check_desc(desc);
  if (st) return st;
  if (check_tensor(q) || check_tensor(k) || !lse || !energy) return CBA_EINVAL;
  if ((v == nullptr) != (o == nullptr)) return CBA_EINVAL;
  if (v && (check_tensor(v) || check_tensor(o))) return CBA_EINVAL;
  if ((reinterpret_cast<uintptr_t>(lse) & 3u) || (reinterpret_cast<uintptr_t>(energy) & 3u)) return CBA_EINVAL;
  AttnParams p = make_params(desc);
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.energy = energy;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (desc->dtype != CBA_DTYPE_BF16) {
    // fp32: the two sweeps (no workspace needed).
    hipError_t e = run_attention(p, desc, /*with_pv=*/v != nullptr, s);
    if (e != hipSuccess) return from_hip(e);
    return from_hip(cba::launch_energy_f32(p, desc->head_dim, desc->block, s));
  }
  const int64_t need = (int64_t)desc->batch * desc->heads * p.nb * p.nb * desc->block * (int64_t)sizeof(float);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 15u) || workspace_bytes < 0) return CBA_EINVAL;
  // A workspace smaller than the whole problem's runs the work in several launches
  // over contiguous (batch item, head, query block) ranges; too small for one
  // workgroup's rows is refused before anything is enqueued.
  const hipError_t e = cba::launch_energy1_bf16(p, desc->head_dim, desc->block, static_cast<float*>(workspace),
                                                workspace_bytes >= need ? -1 : workspace_bytes, s);
  if (e == hipErrorInvalidValue) return CBA_ECAPACITY;
  return from_hip(e);
}

CBA_API cba_status select_blocks_by_energy(const float* energy, int32_t n_draws, int32_t heads, int32_t nb,
                                           double tau, double rho, int32_t force_diag,
                                           int32_t n_dense_prefix_blocks, uint8_t* mask, int32_t* votes,
                                           cba_stream_t stream) {
  if (!energy || !mask) return CBA_EINVAL;
  if (n_draws < 1 || heads < 1 || nb < 1 || nb > 4096) return CBA_EINVAL;
  if ((int64_t)heads * nb > INT32_MAX) return CBA_EINVAL;
  if (!std::isfinite(tau) || !std::isfinite(rho) || tau < 0.0) return CBA_EINVAL;
  if (n_dense_prefix_blocks < 0 || n_dense_prefix_blocks > nb) return CBA_EINVAL;
  cba::TauTable taus{};
  taus.t[0] = tau;
  return from_hip(cba::launch_select(energy, n_draws, heads, nb, taus, rho, force_diag != 0, n_dense_prefix_blocks,
                                     mask, votes, reinterpret_cast<hipStream_t>(stream)));
}

CBA_API cba_status select_blocks_by_energy_heads(const float* energy, int32_t n_draws, int32_t heads, int32_t nb,
                                                 const double* tau_heads, double rho, int32_t force_diag,
                                                 int32_t n_dense_prefix_blocks, uint8_t* mask, int32_t* votes,
                                                 cba_stream_t stream) {
  if (!energy || !mask || !tau_heads) return CBA_EINVAL;
  if (n_draws < 1 || heads < 1 || heads > cba::kMaxTauHeads || nb < 1 || nb > 4096) return CBA_EINVAL;
  if (!std::isfinite(rho) || n_dense_prefix_blocks < 0 || n_dense_prefix_blocks > nb) return CBA_EINVAL;
  cba::TauTable taus{};
  taus.per_head = 1;
  for (int h = 0; h < heads; ++h) {
    if (!std::isfinite(tau_heads[h]) || tau_heads[h] < 0.0) return CBA_EINVAL;
    taus.t[h] = tau_heads[h];
  }
  return from_hip(cba::launch_select(energy, n_draws, heads, nb, taus, rho, force_diag != 0, n_dense_prefix_blocks,
                                     mask, votes, reinterpret_cast<hipStream_t>(stream)));
}

CBA_API cba_status block_energy_from_lse(const cba_attn_desc* desc, const void* q, const void* k, const float* lse,
                                         float* energy, cba_stream_t stream) {
  cba_status st = check_desc(desc);
  if (st) return st;
  if (check_tensor(q) || check_tensor(k) || !lse || !energy) return CBA_EINVAL;
  if ((reinterpret_cast<uintptr_t>(lse) & 3u) || (reinterpret_cast<uintptr_t>(energy) & 3u)) return CBA_EINVAL;
  AttnParams p = make_params(desc);
  p.q = q;
  p.k = k;
  p.lse = const_cast<float*>(lse);  // read only by the energy sweep
  p.energy = energy;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return from_hip(desc->dtype == CBA_DTYPE_BF16 ? cba::launch_energy_bf16(p, desc->head_dim, desc->block, s)
                                                : cba::launch_energy_f32(p, desc->head_dim, desc->block, s));
}

CBA_API cba_status build_block_csr(const uint8_t* mask, int32_t n_rows, int32_t nkb, int32_t* row_ptr,
                                   int32_t* col_idx, int64_t col_idx_capacity, int32_t* work_order,
                                   cba_stream_t stream) {
  if (!mask || !row_ptr || n_rows < 1 || nkb < 1) return CBA_EINVAL;
  if ((int64_t)n_rows * nkb > INT32_MAX) return CBA_EINVAL;  // nnz must fit int32
  if (col_idx && col_idx_capacity < 0) return CBA_EINVAL;
  return from_hip(cba::launch_csr(mask, n_rows, nkb, row_ptr, col_idx, col_idx ? col_idx_capacity : 0, work_order,
                                  reinterpret_cast<hipStream_t>(stream)));
}

CBA_API cba_status sparse_attn_fwd(const cba_attn_desc* desc, const void* q, const void* k, const void* v,
                                   const int32_t* row_ptr, const int32_t* col_idx, int64_t col_idx_len,
                                   const int32_t* work_order, const uint8_t* rep_heads, int32_t anchor_stride,
                                   int32_t fuse_broadcast, void* o, float* lse, cba_stream_t stream) {
  cba_status st = check_desc(desc);
  if (st) return st;
  if (check_tensor(q) || check_tensor(k) || check_tensor(v) || check_tensor(o)) return CBA_EINVAL;
  if (!row_ptr || col_idx_len < 0 || (col_idx_len > 0 && !col_idx)) return CBA_EINVAL;
  AttnParams p = make_params(desc);
  if ((st = set_rep(p, desc, rep_heads, anchor_stride))) return st;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.row_ptr = row_ptr;
  p.col_idx = col_idx;
  p.col_len = col_idx_len;
  p.work_order = work_order;
  p.fuse_broadcast = fuse_broadcast != 0;
  return from_hip(run_attention(p, desc, /*with_pv=*/true, reinterpret_cast<hipStream_t>(stream)));
}

CBA_API cba_status order_heavy_rows_first(const int32_t* row_ptr, int32_t n_rows, int32_t nkb, double factor,
                                          int32_t* work_order, cba_stream_t stream) {
  if (!row_ptr || !work_order || n_rows < 1 || nkb < 1) return CBA_EINVAL;
  if ((int64_t)n_rows * nkb > INT32_MAX || !std::isfinite(factor) || factor < 0.0) return CBA_EINVAL;
  return from_hip(cba::launch_heavy_order(row_ptr, n_rows, nkb, factor, work_order,
                                          reinterpret_cast<hipStream_t>(stream)));
}

CBA_API cba_status build_block_intervals(const uint8_t* mask, int32_t n_rows, int32_t nkb, int32_t* iv_ptr,
                                         uint32_t* ivs, int64_t iv_capacity, cba_stream_t stream) {
  if (!mask || !iv_ptr || n_rows < 1 || nkb < 1 || nkb > 65535) return CBA_EINVAL;
  if ((int64_t)n_rows * nkb > INT32_MAX) return CBA_EINVAL;  // run counts must fit int32
  if (ivs && iv_capacity < 0) return CBA_EINVAL;
  return from_hip(cba::launch_intervals(mask, n_rows, nkb, iv_ptr, ivs, ivs ? iv_capacity : 0,
                                        reinterpret_cast<hipStream_t>(stream)));
}

CBA_API cba_status sparse_attn_fwd_intervals(const cba_attn_desc* desc, const void* q, const void* k,
                                             const void* v, const int32_t* iv_ptr, const uint32_t* ivs,
                                             int64_t iv_len, const int32_t* work_order, const uint8_t* rep_heads,
                                             int32_t anchor_stride, int32_t fuse_broadcast, void* o, float* lse,
                                             cba_stream_t stream) {
  cba_status st = check_desc(desc);
  if (st) return st;
  if (check_tensor(q) || check_tensor(k) || check_tensor(v) || check_tensor(o)) return CBA_EINVAL;
  if (!iv_ptr || iv_len < 0 || (iv_len > 0 && !ivs)) return CBA_EINVAL;
  AttnParams p = make_params(desc);
  if ((st = set_rep(p, desc, rep_heads, anchor_stride))) return st;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.row_ptr = iv_ptr;
  // A non-null runs pointer selects interval mode; with iv_len == 0 no row has a run
  // and the pointer is never read, so any device address serves.
  p.ivs = iv_len > 0 ? ivs : reinterpret_cast<const uint32_t*>(iv_ptr);
  p.col_len = iv_len;
  p.work_order = work_order;
  p.fuse_broadcast = fuse_broadcast != 0;
  return from_hip(run_attention(p, desc, /*with_pv=*/true, reinterpret_cast<hipStream_t>(stream)));
}

CBA_API cba_status rep_row_broadcast(const cba_attn_desc* desc, void* o, const uint8_t* rep_heads,
                                     int32_t anchor_stride, cba_stream_t stream) {
  cba_status st = check_desc(desc);
  if (st) return st;
  if (check_tensor(o) || !rep_heads) return CBA_EINVAL;
  AttnParams p = make_params(desc);
  if ((st = set_rep(p, desc, rep_heads, anchor_stride))) return st;
  p.o = o;
  if (!p.has_rep || anchor_stride == 1) return CBA_OK;  // nothing to copy
  return from_hip(
      cba::launch_broadcast(p, desc->head_dim, elem_bytes(desc->dtype), reinterpret_cast<hipStream_t>(stream)));
}

CBA_API cba_status dense_attn_fwd(const cba_attn_desc* desc, const void* q, const void* k, const void* v, void* o,
                                  float* lse, cba_stream_t stream) {
  cba_status st = check_desc(desc);
  if (st) return st;
  if (check_tensor(q) || check_tensor(k) || check_tensor(v) || check_tensor(o)) return CBA_EINVAL;
  AttnParams p = make_params(desc);
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  return from_hip(run_attention(p, desc, /*with_pv=*/true, reinterpret_cast<hipStream_t>(stream)));
}

CBA_API cba_status spatial_rep_similarity(const cba_attn_desc* desc, const void* q, const void* k,
                                          const float* lse, int32_t anchor_stride, float* token_cos,
                                          float* head_sim, cba_stream_t stream) {
  cba_status st = check_desc(desc, /*uses_block=*/false);
  if (st) return st;
  if (check_tensor(q) || check_tensor(k)) return CBA_EINVAL;
  for (const void* t : {(const void*)lse, (const void*)token_cos, (const void*)head_sim})
    if (!t || (reinterpret_cast<uintptr_t>(t) & 3u)) return CBA_EINVAL;
  if ((int64_t)desc->grid_f * desc->grid_h * desc->grid_w == 0) return CBA_EINVAL;  // needs a token grid
  if (anchor_stride < 2 || desc->grid_h < 2) return CBA_EINVAL;                      // no follower rows
  const AttnParams a = make_params(desc);
  cba::RepParams p{};
  p.q = q;
  p.k = k;
  p.lse = lse;
  p.token_cos = token_cos;
  p.head_sim = head_sim;
  p.sb = a.sb;
  p.sh = a.sh;
  p.sn = a.sn;
  p.batch = a.batch;
  p.heads = a.heads;
  p.n = a.n;
  p.n_prefix = a.n_prefix;
  p.gf = a.gf;
  p.gh = a.gh;
  p.gw = a.gw;
  p.stride = anchor_stride;
  p.c = a.c;
  const bool bf16 = desc->dtype == CBA_DTYPE_BF16;
  const int64_t items =
      cba::rep_grid(p.batch, p.heads, p.gf, p.gh, p.gw, p.stride, bf16, &p.n_groups, &p.n_sub, &p.n_chunks);
  if (items > INT32_MAX) return CBA_EINVAL;
  return from_hip(cba::launch_rep_similarity(p, desc->head_dim, bf16, reinterpret_cast<hipStream_t>(stream)));
}

CBA_API cba_status select_rep_heads(const float* head_sim, int32_t n_draws, int32_t heads, double gamma,
                                    uint8_t* rep_heads, cba_stream_t stream) {
  if (!head_sim || !rep_heads || (reinterpret_cast<uintptr_t>(head_sim) & 3u)) return CBA_EINVAL;
  if (n_draws < 1 || heads < 1 || !std::isfinite(gamma)) return CBA_EINVAL;
  if ((int64_t)n_draws * heads > INT32_MAX) return CBA_EINVAL;
  return from_hip(cba::launch_rep_flags(head_sim, n_draws, heads, gamma, rep_heads,
                                        reinterpret_cast<hipStream_t>(stream)));
}

CBA_API const char* cba_status_str(cba_status status) {
  switch (status) {
    case CBA_OK: return "ok";
    case CBA_EINVAL: return "invalid argument";
    case CBA_EUNSUPPORTED: return "unsupported dtype, head_dim or block";
    case CBA_EHIP: return "HIP launch failed";
    case CBA_ECAPACITY: return "buffer too small";
    default: return "unknown status";
  }
}

CBA_API int32_t cba_version(void) { return 100; }
