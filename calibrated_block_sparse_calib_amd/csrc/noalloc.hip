// calib_block_energy_ws for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
// one-pass energy kernel keeps its per-(row, key block) log-sums in a fixed
// device array of this library instead of a caller workspace.
//
// The array is a file-scope device variable: every GPU the library runs on holds
// its own copy, of kScratchBytes, from the first call on that GPU until the
// process ends.  Host code never passes the variable's name to a kernel (on the
// host the name is only a stand-in); it looks up each device's address once,
// with hipGetSymbolAddress, and passes that address.  Calls on one GPU share its
// array: calls that overlap in time on one GPU (two streams, two threads) race on
// it and must be serialised by the caller.  The kernels write every workspace
// entry they read, so the array needs no clearing between calls.
#include <mutex>

#include "api_checks.h"

namespace {

using namespace cba::abi;

constexpr int64_t kScratchBytes = (int64_t)256 << 20;  // 256 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's copy of `scratch`, looked up on the
// first call on that device (with it current) and kept.
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

CBA_API cba_status calib_block_energy_noalloc(const cba_attn_desc* desc, const void* q, const void* k,
                                              const void* v, void* o, float* lse, float* energy,
                                              cba_stream_t stream) {
  cba_status st = check_desc(desc);
  if (st) return st;
  if (check_tensor(q) || check_tensor(k) || !lse || !energy) return CBA_EINVAL;
  if ((v == nullptr) != (o == nullptr)) return CBA_EINVAL;
  if (v && (check_tensor(v) || check_tensor(o))) return CBA_EINVAL;
  if ((reinterpret_cast<uintptr_t>(lse) & 3u) || (reinterpret_cast<uintptr_t>(energy) & 3u)) return CBA_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // The scratch address is the current device's: the stream must belong to it.
  if (s) {
    int cur = -1, sdev = -1;
    if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(s, &sdev) != hipSuccess) {
      return from_hip(hipErrorInvalidValue);
    }
    if (cur != sdev) return CBA_EINVAL;
  }
  cba::AttnParams p = make_params(desc);
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.energy = energy;
  if (desc->dtype != CBA_DTYPE_BF16) {
    // fp32: the two sweeps, which need no workspace (as calib_block_energy_ws).
    hipError_t e = run_attention(p, desc, /*with_pv=*/v != nullptr, s);
    if (e != hipSuccess) return from_hip(e);
    return from_hip(cba::launch_energy_f32(p, desc->head_dim, desc->block, s));
  }
  void* ws = nullptr;
  hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return from_hip(e);
  e = cba::launch_energy1_bf16(p, desc->head_dim, desc->block, static_cast<float*>(ws), kScratchBytes, s);
  if (e == hipErrorInvalidValue) return CBA_ECAPACITY;  // one workgroup's rows exceed the array; nothing enqueued
  return from_hip(e);
}
