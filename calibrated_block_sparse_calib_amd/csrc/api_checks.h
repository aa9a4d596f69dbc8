// Host-side argument checks and parameter packing shared by the C-ABI entry
// points (api.hip, noalloc.hip).  Not part of the public interface.
#pragma once

#include <cmath>
#include <cstdint>

#include "../../include/calibattn.h"
#include "cba_internal.h"

#define CBA_API extern "C" __attribute__((visibility("default")))

namespace cba {
namespace abi {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int elem_bytes(int dtype) { return dtype == CBA_DTYPE_BF16 ? 2 : 4; }

// Shape, stride and dtype checks shared by every attention-shaped call.  A call
// that does not use blocks (uses_block = false) ignores desc->block.
inline cba_status check_desc(const cba_attn_desc* d, bool uses_block = true) {
  if (!d) return CBA_EINVAL;
  if (d->dtype != CBA_DTYPE_F32 && d->dtype != CBA_DTYPE_BF16) return CBA_EUNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return CBA_EUNSUPPORTED;
  if (uses_block && d->block != 32 && d->block != 64 && d->block != 128) return CBA_EUNSUPPORTED;
  if (d->batch < 1 || d->heads < 1 || d->seq_len < 1) return CBA_EINVAL;
  if (d->n_prefix < 0 || d->n_prefix > d->seq_len) return CBA_EINVAL;
  if (uses_block && d->n_prefix % d->block != 0) return CBA_EINVAL;
  if (d->grid_f < 0 || d->grid_h < 0 || d->grid_w < 0) return CBA_EINVAL;
  const int64_t grid = (int64_t)d->grid_f * d->grid_h * d->grid_w;
  if (grid != 0 && grid != (int64_t)d->seq_len - d->n_prefix) return CBA_EINVAL;
  if (!std::isfinite(d->scale)) return CBA_EINVAL;
  if (d->stride_n < d->head_dim || d->stride_h < 0 || d->stride_b < 0) return CBA_EINVAL;
  const int eb = elem_bytes(d->dtype);
  if ((d->stride_n * eb) % 16 || (d->stride_h * eb) % 16 || (d->stride_b * eb) % 16) return CBA_EINVAL;
  if (uses_block) {
    const int64_t nb = ((int64_t)d->seq_len + d->block - 1) / d->block;
    if ((int64_t)d->heads * nb * d->batch > INT32_MAX) return CBA_EINVAL;
  }
  if ((int64_t)d->batch * d->heads > 65535) return CBA_EINVAL;
  return CBA_OK;
}

inline cba_status check_tensor(const void* p) { return (p && aligned16(p)) ? CBA_OK : CBA_EINVAL; }

inline AttnParams make_params(const cba_attn_desc* d) {
  AttnParams p{};
  p.batch = d->batch;
  p.heads = d->heads;
  p.n = d->seq_len;
  p.nb = d->block > 0 ? (d->seq_len + d->block - 1) / d->block : 0;
  p.n_rows = d->heads * p.nb;
  p.n_prefix = d->n_prefix;
  p.gf = d->grid_f;
  p.gh = d->grid_h;
  p.gw = d->grid_w;
  p.sb = d->stride_b;
  p.sh = d->stride_h;
  p.sn = d->stride_n;
  const float scale = d->scale == 0.f ? 1.0f / std::sqrt((float)d->head_dim) : d->scale;
  p.c = scale * cba::kLog2e;
  p.anchor_stride = 1;
  return p;
}

// Packs the host repetition flags; fails when repetition is asked for without a
// token grid or beyond the supported head count.
inline cba_status set_rep(AttnParams& p, const cba_attn_desc* d, const uint8_t* rep_heads, int32_t anchor_stride) {
  if (anchor_stride < 1) return CBA_EINVAL;
  p.anchor_stride = anchor_stride;
  if (!rep_heads) return CBA_OK;
  bool any = false;
  for (int h = 0; h < d->heads; ++h) any |= rep_heads[h] != 0;
  if (!any) return CBA_OK;
  if (d->heads > cba::kMaxRepHeads) return CBA_EINVAL;
  if ((int64_t)d->grid_f * d->grid_h * d->grid_w == 0) return CBA_EINVAL;
  for (int h = 0; h < d->heads; ++h)
    if (rep_heads[h]) p.rep_bits[h >> 5] |= 1u << (h & 31);
  p.has_rep = 1;
  return CBA_OK;
}

inline cba_status from_hip(hipError_t e) {
  if (e == hipSuccess) return CBA_OK;
  (void)hipGetLastError();  // clear the sticky launch error for the caller
  return CBA_EHIP;
}

// Dense when p.row_ptr is null.
inline hipError_t run_attention(const AttnParams& p, const cba_attn_desc* d, bool with_pv, hipStream_t s) {
  return d->dtype == CBA_DTYPE_BF16 ? cba::launch_attn_bf16(p, d->head_dim, d->block, with_pv, s)
                                    : cba::launch_attn_f32(p, d->head_dim, d->block, with_pv, s);
}

}  // namespace abi
}  // namespace cba
