// fp32 attention kernels: the full-precision path (inputs, products and softmax in
// fp32 on the vector ALUs).  It serves fp32 workloads, where results must agree
// with an fp64 evaluation to about 1e-5, and is not tuned for speed.
//
// One workgroup per (query block, batch item), one thread per computed query row;
// K and V are staged through LDS 32 keys at a time and every thread runs its own
// online softmax.
#include "cba_internal.h"

namespace cba {
namespace {

constexpr int TK = 32;  // keys per LDS tile

template <int D, int B, bool PV>
__global__ __launch_bounds__(B) void attn_f32_kernel(AttnParams p) {
  __shared__ float ks[TK][D + 1];
  __shared__ float vs[PV ? TK : 1][D + 1];
  __shared__ int rowlist[B];
  __shared__ int wcnt[2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int item = blockIdx.x;
  const int it = item / p.batch, b = item - it * p.batch;
  const int row = p.work_order ? p.work_order[it] : it;
  if (row < 0 || row >= p.n_rows) return;
  const int h = row / p.nb, qb = row - h * p.nb;
  const int q0 = qb * B;
  const bool rep = rep_head(p, h);

  int M;
  if (!rep) {
    M = min(B, p.n - q0);
  } else {
    // Text rows and anchor image rows (y % stride == 0), compacted in order.
    bool flag = false;
    const int tok = q0 + tid;
    if (tok < p.n) {
      if (tok < p.n_prefix) {
        flag = true;
      } else {
        const int y = ((tok - p.n_prefix) / p.gw) % p.gh;
        flag = (y % p.anchor_stride) == 0;
      }
    }
    const uint64_t bal = __ballot(flag);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wcnt[wave] = __popcll(bal);
    __syncthreads();
    const int off = wave > 0 ? wcnt[0] : 0;
    M = wcnt[0] + (B > 64 ? wcnt[1] : 0);
    if (flag) rowlist[off + before] = tid;
    __syncthreads();
  }

  const int64_t head_off = (int64_t)b * p.sb + (int64_t)h * p.sh;
  const float* qg = static_cast<const float*>(p.q) + head_off;
  const float* kg = static_cast<const float*>(p.k) + head_off;
  const float* vg = PV ? static_cast<const float*>(p.v) + head_off : nullptr;

  const bool valid = tid < M;
  const int qtok = q0 + (rep ? (valid ? rowlist[tid] : 0) : tid);
  float q[D], o[PV ? D : 1];
#pragma unroll
  for (int d = 0; d < D; ++d) q[d] = valid ? qg[(int64_t)qtok * p.sn + d] : 0.f;
#pragma unroll
  for (int d = 0; d < (PV ? D : 1); ++d) o[d] = 0.f;
  float m = -INFINITY, l = 0.f;

  const bool dense = p.row_ptr == nullptr;  // no list: every key block
  int beg = 0, nblk = p.nb;
  if (!dense) {
    beg = max(p.row_ptr[row], 0);
    const int64_t end = min((int64_t)p.row_ptr[row + 1], p.col_len);
    nblk = (int)max((int64_t)0, end - beg);
  }
  // Interval skip list: [beg, beg + nblk) are runs (first | count << 16); a cursor
  // (run iv_j, offset iv_off) walks their blocks in order.
  const int iv_end = beg + nblk;
  int iv_j = beg, iv_off = 0, total = nblk;
  if (p.ivs) {
    total = 0;
    for (int j = beg; j < iv_end; ++j) total += (int)(p.ivs[j] >> 16);
  }
  for (int bi = 0; bi < total; ++bi) {
    int kb;
    if (p.ivs) {
      while (iv_j < iv_end && iv_off >= (int)(p.ivs[iv_j] >> 16)) {
        ++iv_j;
        iv_off = 0;
      }
      kb = iv_j < iv_end ? (int)(p.ivs[iv_j] & 0xffffu) + iv_off : -1;
      ++iv_off;
    } else {
      kb = dense ? bi : p.col_idx[beg + bi];
    }
    if (kb < 0 || kb >= p.nb) continue;
    for (int sub = 0; sub < B / TK; ++sub) {
      const int k0 = kb * B + sub * TK;
      if (k0 >= p.n) break;
      __syncthreads();
      for (int idx = tid; idx < TK * D; idx += B) {
        const int r = idx / D, c = idx - r * D;
        const int key = k0 + r;
        ks[r][c] = key < p.n ? kg[(int64_t)key * p.sn + c] : 0.f;
        if (PV) vs[r][c] = key < p.n ? vg[(int64_t)key * p.sn + c] : 0.f;
      }
      __syncthreads();
      if (!valid) continue;
      float s[TK];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < TK; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) acc = fmaf(q[d], ks[j][d], acc);
        s[j] = (k0 + j < p.n) ? acc * p.c : -INFINITY;
        mx = fmaxf(mx, s[j]);
      }
      const float m_new = fmaxf(m, mx);
      const float alpha = exp2f(m - m_new);
      l *= alpha;
      if (PV) {
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] *= alpha;
      }
      m = m_new;
#pragma unroll
      for (int j = 0; j < TK; ++j) {
        const float pj = exp2f(s[j] - m);
        l += pj;
        if (PV) {
#pragma unroll
          for (int d = 0; d < D; ++d) o[d] = fmaf(pj, vs[j][d], o[d]);
        }
      }
    }
  }
  if (!valid) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const float lse_val = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
  int n_follow = 0;
  if (rep && qtok >= p.n_prefix) {
    const int y = ((qtok - p.n_prefix) / p.gw) % p.gh;
    n_follow = min(p.anchor_stride - 1, p.gh - 1 - y);
  }
  if (PV && p.o) {
    float* og = static_cast<float*>(p.o) + head_off;
    const int n_copies = p.fuse_broadcast ? n_follow : 0;
    for (int cp = 0; cp <= n_copies; ++cp) {
      float* orow = og + (int64_t)(qtok + cp * p.gw) * p.sn;
#pragma unroll
      for (int d = 0; d < D; ++d) orow[d] = o[d] * inv;
    }
  }
  if (p.lse) {
    float* lg = p.lse + ((int64_t)b * p.heads + h) * p.n;
    for (int cp = 0; cp <= n_follow; ++cp) lg[qtok + cp * p.gw] = lse_val;
  }
}

// Block energy sweep 2 in fp32: each thread sums exp(s_ij - lse_i) of its row over
// a key block; the rows' partial sums are then added in row order by one thread.
template <int D, int B>
__global__ __launch_bounds__(B) void energy_f32_kernel(AttnParams p) {
  __shared__ float ks[TK][D + 1];
  __shared__ float red[B];
  const int tid = threadIdx.x;
  const int item = blockIdx.x;
  const int it = item / p.batch, b = item - it * p.batch;
  const int h = it / p.nb, qb = it - h * p.nb;
  const int q0 = qb * B;
  const bool valid = q0 + tid < p.n;
  const int qtok = q0 + tid;
  const int64_t head_off = (int64_t)b * p.sb + (int64_t)h * p.sh;
  const float* qg = static_cast<const float*>(p.q) + head_off;
  const float* kg = static_cast<const float*>(p.k) + head_off;
  float q[D];
#pragma unroll
  for (int d = 0; d < D; ++d) q[d] = valid ? qg[(int64_t)qtok * p.sn + d] : 0.f;
  const float lse2 = valid ? p.lse[((int64_t)b * p.heads + h) * p.n + qtok] * kLog2e : 0.f;
  float* eg = p.energy + (((int64_t)b * p.heads + h) * p.nb + qb) * p.nb;

  for (int kb = 0; kb < p.nb; ++kb) {
    float esum = 0.f;
    for (int sub = 0; sub < B / TK; ++sub) {
      const int k0 = kb * B + sub * TK;
      if (k0 >= p.n) break;
      __syncthreads();
      for (int idx = tid; idx < TK * D; idx += B) {
        const int r = idx / D, c = idx - r * D;
        const int key = k0 + r;
        ks[r][c] = key < p.n ? kg[(int64_t)key * p.sn + c] : 0.f;
      }
      __syncthreads();
      if (!valid) continue;
#pragma unroll 4
      for (int j = 0; j < TK; ++j) {
        if (k0 + j >= p.n) break;
        float acc = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) acc = fmaf(q[d], ks[j][d], acc);
        esum += exp2f(acc * p.c - lse2);
      }
    }
    red[tid] = valid ? esum : 0.f;
    __syncthreads();
    if (tid == 0) {
      float e = 0.f;
      for (int t = 0; t < B; ++t) e += red[t];
      eg[kb] = e;
    }
  }
}

template <int D, int B>
hipError_t launch_attn_t(const AttnParams& p, bool with_pv, hipStream_t stream) {
  void (*kern)(AttnParams) = with_pv ? attn_f32_kernel<D, B, true> : attn_f32_kernel<D, B, false>;
  AttnParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel((const void*)kern, dim3((unsigned)((int64_t)p.n_rows * p.batch)), dim3(B), args, 0,
                         stream);
}

template <int D, int B>
hipError_t launch_energy_t(const AttnParams& p, hipStream_t stream) {
  AttnParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel((const void*)energy_f32_kernel<D, B>,
                         dim3((unsigned)((int64_t)p.heads * p.nb * p.batch)), dim3(B), args, 0, stream);
}

}  // namespace

hipError_t launch_attn_f32(const AttnParams& p, int head_dim, int block, bool with_pv, hipStream_t stream) {
#define CBA_CASE(D, B) \
  if (head_dim == D && block == B) return launch_attn_t<D, B>(p, with_pv, stream);
  CBA_CASE(64, 32) CBA_CASE(64, 64) CBA_CASE(64, 128)
  CBA_CASE(128, 32) CBA_CASE(128, 64) CBA_CASE(128, 128)
#undef CBA_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_energy_f32(const AttnParams& p, int head_dim, int block, hipStream_t stream) {
#define CBA_CASE(D, B) \
  if (head_dim == D && block == B) return launch_energy_t<D, B>(p, stream);
  CBA_CASE(64, 32) CBA_CASE(64, 64) CBA_CASE(64, 128)
  CBA_CASE(128, 32) CBA_CASE(128, 64) CBA_CASE(128, 128)
#undef CBA_CASE
  return hipErrorInvalidValue;
}

}  // namespace cba
