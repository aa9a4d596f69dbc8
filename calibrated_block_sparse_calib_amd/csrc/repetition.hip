// Spatial-repetition detection for the calibration stage: for every follower grid
// token (f, y, x), y % s != 0, the cosine similarity between its row of dense
// attention probabilities and that of its anchor (f, s*floor(y/s), x); then the
// per-head mean, and the repetition flags from the means over calibration inputs.
//
// Work decomposition (bf16): one workgroup per (batch item and head, row group,
// follower sub-group, chunk of 2 x 32 (frame, column) pairs).  For each 32-pair
// column group, one wave computes the anchor row of the row group and NWV-1 waves
// up to NWV-1 of its follower rows, all for the same 32 (frame, column) pairs, so
// lane l of each of those waves holds the same column and, in the MFMA accumulator
// layout, the same keys.  All waves of the workgroup walk the whole key sequence
// together, sharing each K tile staged in LDS (double buffered, one barrier per
// step) between both column groups.  Per step the anchor wave writes its 64 x 32
// probabilities to its group's LDS exchange buffer; the follower waves keep their own
// probabilities in registers and combine them with the anchor's one step later,
// after the next barrier, so no extra barrier is needed.  Scores are computed
// transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16.
//
// The probabilities are exp(s_ij - lse_i) with the caller's log-sum-exp; the
// cosine does not depend on that per-row factor.  Dot products and squared norms
// accumulate in fp32, one partial sum per step added to the running total.
#include "cba_internal.h"
#include "mfma_util.h"

namespace cba {
namespace {

using namespace dev;

constexpr int kKT = 64;  // keys per step (bf16)

template <int D, int NWV, bool BUF>
__global__ __launch_bounds__(kRepGroups * NWV * 64, 2) void rep_sim_bf16_kernel(RepParams p) {
  constexpr int KS = D / 16, TILE = kKT * D, NW = kRepGroups * NWV;
  __shared__ __attribute__((aligned(16))) bfraw k0s[TILE], k1s[TILE];
  __shared__ __attribute__((aligned(16))) float xch[kRepGroups][2][8 * 64 * 4];  // [group][buffer][float4 j][lane]
  __shared__ float anrm[kRepGroups][32];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5;
  const int wave = tid >> 6, gl = wave / NWV, wl = wave - gl * NWV;  // column group, wave in the group
  int item = blockIdx.x;
  const int chunk = item % p.n_chunks;
  item /= p.n_chunks;
  const int sub = item % p.n_sub;
  item /= p.n_sub;
  const int grp = item % p.n_groups;
  const int bh = item / p.n_groups;
  const int b = bh / p.heads, h = bh - b * p.heads;

  const int y0 = grp * p.stride;
  const int rows = min(p.stride, p.gh - y0);
  const int r = wl == 0 ? 0 : 1 + sub * (NWV - 1) + (wl - 1);
  const bool active = r < rows;
  const int npairs = p.gf * p.gw;
  const int u = (chunk * kRepGroups + gl) * 32 + (lane & 31);
  const bool u_valid = u < npairs;
  const int uu = u_valid ? u : npairs - 1;  // surplus lanes recompute the last column
  const int f = uu / p.gw, x = uu - f * p.gw;
  const int tok = p.n_prefix + (f * p.gh + y0 + (active ? r : 0)) * p.gw + x;

  const int64_t head_off = (int64_t)b * p.sb + (int64_t)h * p.sh;
  const bfraw* qg = static_cast<const bfraw*>(p.q) + head_off;
  const bfraw* kg = static_cast<const bfraw*>(p.k) + head_off;
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qf[ks] = *reinterpret_cast<const bf16x8*>(qg + (int64_t)tok * p.sn + ks * 16 + g * 8);
  const int64_t row_base = (int64_t)bh * p.n;
  const float lse2 = p.lse[row_base + tok] * kLog2e;

  const int nsteps = (p.n + kKT - 1) / kKT;
  constexpr int LPW = kKT / (64 / (D / 8)) / NW;
  int voff[LPW];
  if (BUF) tile_lane_offsets<D, kKT, NW>((int)(p.sn * 2), voff);
  const TileSrc ksrc = tile_src<D>(kg, p.n, p.sn);
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  auto load = [&](int k0, bfraw* kdst) __attribute__((always_inline)) {
    if (BUF) load_tile_buf(ksrc, k0, voff, LPW, kdst + wv * LPW * 512);
    else load_tile<D, kKT, NW>(kg, p.sn, p.n, k0, kdst);
  };

  float pv[32];    // this step's probabilities (follower waves: last step's, until combined)
  float dot = 0.f, nrm = 0.f;
  auto combine = [&](int buf) __attribute__((always_inline)) {
    // pv holds this wave's probabilities of the step whose anchor values are in xch[buf].
    const float4* src = reinterpret_cast<const float4*>(xch[gl][buf]);
    float d_step = 0.f, n_step = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float4 a = src[j * 64 + lane];
      d_step = fmaf(pv[4 * j + 0], a.x, d_step);
      d_step = fmaf(pv[4 * j + 1], a.y, d_step);
      d_step = fmaf(pv[4 * j + 2], a.z, d_step);
      d_step = fmaf(pv[4 * j + 3], a.w, d_step);
#pragma unroll
      for (int e = 0; e < 4; ++e) n_step = fmaf(pv[4 * j + e], pv[4 * j + e], n_step);
    }
    dot += d_step;
    nrm += n_step;
  };

  load(0, k0s);
  for (int s = 0; s < nsteps; ++s) {
    const bfraw* kt = (s & 1) ? k1s : k0s;
    bfraw* kn = (s & 1) ? k0s : k1s;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // Follower waves first fold in the previous step: its anchor values became
    // visible at this barrier.
    if (wl > 0 && active && s > 0) combine((s - 1) & 1);
    if (s + 1 < nsteps) load((s + 1) * kKT, kn);
    if (!active) continue;
    const int k0 = s * kKT;
    f32x16 sacc[2];
    qk_step<D, kKT>(kt, qf, sacc);
    if (k0 + kKT > p.n) mask_ragged<2>(sacc, p.n, k0);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) pv[t * 16 + i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][i], p.c, -lse2));
    if (wl == 0) {
      float4* dst = reinterpret_cast<float4*>(xch[gl][s & 1]);
      float n_step = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        dst[j * 64 + lane] = make_float4(pv[4 * j], pv[4 * j + 1], pv[4 * j + 2], pv[4 * j + 3]);
#pragma unroll
        for (int e = 0; e < 4; ++e) n_step = fmaf(pv[4 * j + e], pv[4 * j + e], n_step);
      }
      nrm += n_step;
    }
  }
  __syncthreads();
  if (wl > 0 && active) combine((nsteps - 1) & 1);
  // Each lane holds half of its column's keys; add the other half's.
  dot += other_half(dot);
  nrm += other_half(nrm);
  if (wl == 0 && lane < 32) anrm[gl][lane] = nrm;
  __syncthreads();
  if (wl > 0 && active && u_valid && g == 0) {
    p.token_cos[row_base + tok] = dot / sqrtf(nrm * anrm[gl][lane]);
  }
}

// fp32 inputs: the full-precision path, not tuned for speed.  One workgroup per
// (batch item and head, row group, follower sub-group, chunk of 64 (frame,
// column) pairs); one thread per query token; wave 0 the anchor row.  K is staged
// 32 keys at a time and the anchor's probabilities pass through LDS.
template <int D, int NWV>
__global__ __launch_bounds__(NWV * 64) void rep_sim_f32_kernel(RepParams p) {
  constexpr int TK = 32;
  __shared__ float ks[TK][D + 1];
  __shared__ float pa[TK][64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int item = blockIdx.x;
  const int chunk = item % p.n_chunks;
  item /= p.n_chunks;
  const int sub = item % p.n_sub;
  item /= p.n_sub;
  const int grp = item % p.n_groups;
  const int bh = item / p.n_groups;
  const int b = bh / p.heads, h = bh - b * p.heads;

  const int y0 = grp * p.stride;
  const int rows = min(p.stride, p.gh - y0);
  const int r = wave == 0 ? 0 : 1 + sub * (NWV - 1) + (wave - 1);
  const bool active = r < rows;
  const int npairs = p.gf * p.gw;
  const int u = chunk * 64 + lane;
  const bool u_valid = u < npairs;
  const int uu = u_valid ? u : npairs - 1;
  const int f = uu / p.gw, x = uu - f * p.gw;
  const int tok = p.n_prefix + (f * p.gh + y0 + (active ? r : 0)) * p.gw + x;

  const int64_t head_off = (int64_t)b * p.sb + (int64_t)h * p.sh;
  const float* qg = static_cast<const float*>(p.q) + head_off;
  const float* kg = static_cast<const float*>(p.k) + head_off;
  float q[D];
#pragma unroll
  for (int d = 0; d < D; ++d) q[d] = qg[(int64_t)tok * p.sn + d];
  const int64_t row_base = (int64_t)bh * p.n;
  const float lse2 = p.lse[row_base + tok] * kLog2e;

  float dot = 0.f, nrm = 0.f;
  for (int k0 = 0; k0 < p.n; k0 += TK) {
    __syncthreads();
    for (int idx = tid; idx < TK * D; idx += NWV * 64) {
      const int rr = idx / D, cc = idx - rr * D;
      const int key = k0 + rr;
      ks[rr][cc] = key < p.n ? kg[(int64_t)key * p.sn + cc] : 0.f;
    }
    __syncthreads();
    float pj[TK];
#pragma unroll
    for (int j = 0; j < TK; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc = fmaf(q[d], ks[j][d], acc);
      pj[j] = (k0 + j < p.n) ? exp2f(acc * p.c - lse2) : 0.f;
    }
    if (wave == 0) {
#pragma unroll
      for (int j = 0; j < TK; ++j) pa[j][lane] = pj[j];
    }
    float d_step = 0.f, n_step = 0.f;
#pragma unroll
    for (int j = 0; j < TK; ++j) n_step = fmaf(pj[j], pj[j], n_step);
    __syncthreads();
    if (wave > 0 && active) {
#pragma unroll
      for (int j = 0; j < TK; ++j) d_step = fmaf(pj[j], pa[j][lane], d_step);
    }
    dot += d_step;
    nrm += n_step;
  }
  __syncthreads();
  if (wave == 0) pa[0][lane] = nrm;
  __syncthreads();
  if (wave > 0 && active && u_valid) p.token_cos[row_base + tok] = dot / sqrtf(nrm * pa[0][lane]);
}

// Mean of token_cos over the follower tokens of one (batch item, head): fp64
// partial sums in a fixed thread order, then a fixed tree.
constexpr int kMeanThreads = 256;

__global__ __launch_bounds__(kMeanThreads) void rep_mean_kernel(RepParams p) {
  __shared__ double red[kMeanThreads];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int s = p.stride;
  const int anchors = (p.gh + s - 1) / s;
  const int nfr = p.gh - anchors;  // follower rows per frame
  const int64_t count = (int64_t)p.gf * nfr * p.gw;
  const float* src = p.token_cos + (int64_t)bh * p.n;
  double acc = 0.0;
  for (int64_t idx = tid; idx < count; idx += kMeanThreads) {
    const int64_t fr = idx / p.gw;
    const int x = (int)(idx - fr * p.gw);
    const int f = (int)(fr / nfr), j = (int)(fr - (int64_t)f * nfr);
    const int y = (j / (s - 1)) * s + j % (s - 1) + 1;  // j-th non-anchor row
    acc += (double)src[p.n_prefix + ((int64_t)f * p.gh + y) * p.gw + x];
  }
  red[tid] = acc;
  __syncthreads();
  for (int w = kMeanThreads / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] += red[tid + w];
    __syncthreads();
  }
  if (tid == 0) p.head_sim[bh] = (float)(red[0] / (double)count);
}

__global__ void rep_flags_kernel(const float* head_sim, int n_draws, int heads, double gamma, uint8_t* flags) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= heads) return;
  double acc = 0.0;
  for (int d = 0; d < n_draws; ++d) acc += (double)head_sim[(int64_t)d * heads + h];
  flags[h] = (acc / (double)n_draws > gamma) ? 1 : 0;
}

template <int D, int NWV>
hipError_t launch_sim_t(const RepParams& p, bool bf16, hipStream_t stream) {
  RepParams arg = p;
  const int64_t items = (int64_t)p.batch * p.heads * p.n_groups * p.n_sub * p.n_chunks;
  if (items < 1 || items > INT32_MAX) return hipErrorInvalidValue;
  void (*kern)(RepParams);
  if (bf16) {
    const bool buf = (int64_t)(p.n + kKT) * p.sn * 2 < ((int64_t)1 << 31);
    kern = buf ? rep_sim_bf16_kernel<D, NWV, true> : rep_sim_bf16_kernel<D, NWV, false>;
  } else {
    kern = rep_sim_f32_kernel<D, NWV>;
  }
  void* args[] = {&arg};
  hipError_t e = hipLaunchKernel((const void*)kern, dim3((unsigned)items), dim3((bf16 ? kRepGroups : 1) * NWV * 64),
                                 args, 0, stream);
  if (e != hipSuccess) return e;
  return hipLaunchKernel((const void*)rep_mean_kernel, dim3((unsigned)(p.batch * p.heads)), dim3(kMeanThreads),
                         args, 0, stream);
}

}  // namespace

hipError_t launch_rep_similarity(const RepParams& p, int head_dim, bool bf16, hipStream_t stream) {
  // Two waves (anchor + one follower) when each group has a single follower row.
  const bool two = p.stride == 2;
  if (head_dim == 64) return two ? launch_sim_t<64, 2>(p, bf16, stream) : launch_sim_t<64, 4>(p, bf16, stream);
  if (head_dim == 128) return two ? launch_sim_t<128, 2>(p, bf16, stream) : launch_sim_t<128, 4>(p, bf16, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_rep_flags(const float* head_sim, int n_draws, int heads, double gamma, uint8_t* flags,
                            hipStream_t stream) {
  const int threads = 256;
  void* args[] = {&head_sim, &n_draws, &heads, &gamma, &flags};
  return hipLaunchKernel((const void*)rep_flags_kernel, dim3((unsigned)((heads + threads - 1) / threads)),
                         dim3(threads), args, 0, stream);
}

}  // namespace cba
