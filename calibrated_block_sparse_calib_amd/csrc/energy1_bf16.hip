// One-pass block energies without V: energies and the log-sum-exp, with QPB query
// blocks per workgroup sharing every K tile (the kernel is in energy1_bf16.h).
#include "energy1_bf16.h"

namespace cba {

hipError_t launch_energy1_k_bf16(const AttnParams& p, int head_dim, int block, float* ws, int64_t ws_bytes,
                                 hipStream_t stream) {
#define CBA_CASE(D, B) \
  if (head_dim == D && block == B) return launch_energy1_q<D, B, energy1_qpb<D, B>(), false>(p, ws, ws_bytes, stream);
  CBA_CASE(64, 32) CBA_CASE(64, 64) CBA_CASE(64, 128)
  CBA_CASE(128, 32) CBA_CASE(128, 64) CBA_CASE(128, 128)
#undef CBA_CASE
  return hipErrorInvalidValue;
}

}  // namespace cba
