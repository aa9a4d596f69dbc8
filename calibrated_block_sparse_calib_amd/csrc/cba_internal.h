// Internal declarations shared by the HIP kernels and the C-ABI layer of
// libcalibattn.so.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cba {

constexpr int kMaxRepHeads = 1024;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Everything an attention-shaped kernel needs: tensor pointers and strides, the
// problem shape, the optional skip list and the repetition-head description.
struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;        // may be null (energy sweep 1 without V)
  float* lse;     // may be null
  float* energy;  // energy sweep 2 output [batch, heads, nb, nb]
  int64_t sb, sh, sn;  // element strides of Q/K/V/O
  int batch, heads, n, nb;
  int n_prefix, gf, gh, gw;
  float c;  // softmax scale * log2(e): scores are handled in base-2 units
  const int32_t* row_ptr;   // skip list: row offsets into col_idx, or into ivs
  const int32_t* col_idx;
  const uint32_t* ivs;      // non-null: runs (first | count << 16) instead of col_idx
  int64_t col_len;          // valid entries of col_idx or ivs
  const int32_t* work_order;
  int n_rows;      // heads * nb
  int anchor_stride;
  int has_rep;
  int fuse_broadcast;
  uint32_t rep_bits[kMaxRepHeads / 32];
};

__host__ __device__ inline bool rep_head(const AttnParams& p, int h) {
  return p.has_rep && ((p.rep_bits[h >> 5] >> (h & 31)) & 1u);
}

// Energy thresholds of the block selection, passed by value to the kernel: one
// for every head (per_head = 0: t[0]) or one per head.
constexpr int kMaxTauHeads = 256;
struct TauTable {
  double t[kMaxTauHeads];
  int per_head;
};

// Spatial-repetition similarity: Q, K and the per-row log-sum-exp of one dense
// pass, the token grid and the anchor stride; outputs per-token cosines and
// per-head means.  n_groups, n_sub and n_chunks describe the launch grid.
struct RepParams {
  const void* q;
  const void* k;
  const float* lse;
  float* token_cos;
  float* head_sim;
  int64_t sb, sh, sn;
  int batch, heads, n;
  int n_prefix, gf, gh, gw;
  int stride;  // anchor stride, >= 2
  float c;     // softmax scale * log2(e)
  int n_groups, n_sub, n_chunks;
};

// Launch grid of the repetition-similarity kernel: (row groups that hold a
// follower row) x (follower sub-groups of NWV - 1 rows) x (chunks of the frame x
// column pairs), per batch item and head.  NWV = 2 waves for stride 2, else 4;
// chunks are 32 pairs wide for bf16 and 64 for fp32.
constexpr int kRepGroups = 2;  // bf16: column groups (of 32 pairs) per workgroup, sharing K tiles

inline int64_t rep_grid(int batch, int heads, int gf, int gh, int gw, int stride, bool bf16, int* n_groups,
                        int* n_sub, int* n_chunks) {
  const int nf = stride == 2 ? 1 : 3;
  const int cw = bf16 ? 32 * kRepGroups : 64;
  *n_groups = (gh - 1 + stride - 1) / stride;
  *n_sub = (stride - 1 + nf - 1) / nf;
  *n_chunks = (int)(((int64_t)gf * gw + cw - 1) / cw);
  return (int64_t)batch * heads * *n_groups * *n_sub * *n_chunks;
}

// Launchers (each enqueues on `stream` and returns the launch status).
// Attention over the key blocks listed in p.row_ptr/p.col_idx, or over every key
// block when p.row_ptr is null (dense).  with_pv = false computes only the LSE.
hipError_t launch_attn_bf16(const AttnParams& p, int head_dim, int block, bool with_pv, hipStream_t stream);
hipError_t launch_energy_bf16(const AttnParams& p, int head_dim, int block, hipStream_t stream);
// One-pass energies with the per-(row, key block) log-sums in ws [batch, heads, nb, nb, block]
// (O too when p.v is set; the _k variant is the case without V).  ws_bytes < 0: ws
// holds all of it; otherwise ws holds ws_bytes and the work goes in several
// launches (hipErrorInvalidValue if one workgroup's rows do not fit).
hipError_t launch_energy1_bf16(const AttnParams& p, int head_dim, int block, float* ws, int64_t ws_bytes,
                               hipStream_t stream);
hipError_t launch_energy1_k_bf16(const AttnParams& p, int head_dim, int block, float* ws, int64_t ws_bytes,
                                 hipStream_t stream);
hipError_t launch_attn_f32(const AttnParams& p, int head_dim, int block, bool with_pv, hipStream_t stream);
hipError_t launch_energy_f32(const AttnParams& p, int head_dim, int block, hipStream_t stream);
hipError_t launch_select(const float* energy, int n_draws, int heads, int nb, const TauTable& taus, double rho,
                         int force_diag, int n_prefix_blocks, uint8_t* mask, int32_t* votes,
                         hipStream_t stream);
hipError_t launch_csr(const uint8_t* mask, int n_rows, int nkb, int32_t* row_ptr, int32_t* col_idx,
                      int64_t capacity, int32_t* work_order, hipStream_t stream);
hipError_t launch_heavy_order(const int32_t* row_ptr, int n_rows, int nkb, double factor, int32_t* work_order,
                              hipStream_t stream);
hipError_t launch_intervals(const uint8_t* mask, int n_rows, int nkb, int32_t* iv_ptr, uint32_t* ivs,
                            int64_t capacity, hipStream_t stream);
hipError_t launch_broadcast(const AttnParams& p, int head_dim, int elem_bytes, hipStream_t stream);
// Per-token cosines then per-head means; p.n_groups/n_sub/n_chunks from rep_grid.
hipError_t launch_rep_similarity(const RepParams& p, int head_dim, bool bf16, hipStream_t stream);
hipError_t launch_rep_flags(const float* head_sim, int n_draws, int heads, double gamma, uint8_t* flags,
                            hipStream_t stream);

}  // namespace cba
