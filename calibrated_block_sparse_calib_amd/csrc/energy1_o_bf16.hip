// One-pass block energies with V: O, the log-sum-exp and the energies, one query
// block per workgroup as the dense pass (the kernel is in energy1_bf16.h).
#include "energy1_bf16.h"

namespace cba {

hipError_t launch_energy1_bf16(const AttnParams& p, int head_dim, int block, float* ws, int64_t ws_bytes,
                               hipStream_t stream) {
  if (!p.v) return launch_energy1_k_bf16(p, head_dim, block, ws, ws_bytes, stream);
#define CBA_CASE(D, B) \
  if (head_dim == D && block == B) return launch_energy1_q<D, B, 1, true>(p, ws, ws_bytes, stream);
  CBA_CASE(64, 32) CBA_CASE(64, 64) CBA_CASE(64, 128)
  CBA_CASE(128, 32) CBA_CASE(128, 64) CBA_CASE(128, 128)
#undef CBA_CASE
  return hipErrorInvalidValue;
}

}  // namespace cba
