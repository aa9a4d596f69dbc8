// bf16 attention kernels for gfx950: block-sparse / dense forward and the
// block-energy sweep.  bf16 operands on the matrix cores (v_mfma_f32_32x32x16_bf16),
// fp32 accumulation and fp32 online softmax.
//
// Work decomposition: one workgroup per (query block, batch item) -- B query
// rows -- with B/32 waves of 32 query rows each.  The workgroup walks the key
// blocks listed for its query block (the skip list of the CalibAtt inference
// stage, zh S2.2B / fr S2C) in steps of KT keys.  Each step stages a K tile and a
// V tile in LDS (double buffered, one barrier per step, the next step's global
// loads in flight during the current step's math).
//
// Per wave and step the scores are computed transposed, S^T = K Q^T, so that
// every lane owns one query row: the row max and row sum of the online softmax
// stay in-lane except for one exchange between the two 32-lane halves.  The
// probabilities are kept in the MFMA accumulator layout and fed straight back as
// the B operand of O^T += V^T P^T; V^T fragments come from the row-major V tile
// through the LDS transpose read (ds_read_b64_tr_b16), with the key order of
// each fragment matched to the order in which the accumulator holds P.
//
// The running maximum is rescaled lazily: the output and sum are rescaled only
// when a row maximum grows by more than 2^8 in base-2 units, so most steps skip
// the rescale.  Numerator and denominator always share the same reference, so
// the result is the exact softmax up to rounding.
#include "cba_internal.h"
#include "mfma_util.h"

namespace cba {
namespace {

using namespace dev;

// One work item: query block qb of head h (row = h * nb + qb) for batch item b.
// Every barrier inside is reached by all threads of the workgroup; the only early
// exits are before the first barrier (uniform) or after the last one.
// The four tile buffers are separate LDS objects, so the compiler can tell that
// the reads of one buffer never alias the asynchronous loads into another and
// does not wait for those loads before reading.
// IV: the skip list is given as runs of consecutive blocks (p.ivs) instead of
// block indices (p.col_idx).
template <int D, int B, bool PV, bool LSE, bool BUF, bool IV>
__device__ __forceinline__ void attn_item(const AttnParams& p, int row, int b, bfraw* k0s, bfraw* k1s,
                                          bfraw* v0s, bfraw* v1s, int* rowlist, int* wcnt) {
  using C = Cfg<D, B>;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5;
  if (row < 0 || row >= p.n_rows) return;
  const int h = row / p.nb, qb = row - h * p.nb;
  const int q0 = qb * B;
  const bool rep = rep_head(p, h);
  const int M = build_rowlist<B, C::NT>(p, q0, rep, rowlist, wcnt);
  // A block of a repetition head with no text or anchor row computes nothing:
  // its rows are followers, written from their anchors' blocks.
  if (M == 0) return;

  const int64_t head_off = (int64_t)b * p.sb + (int64_t)h * p.sh;
  const bfraw* qg = static_cast<const bfraw*>(p.q) + head_off;
  const bfraw* kg = static_cast<const bfraw*>(p.k) + head_off;
  const bfraw* vg = PV ? static_cast<const bfraw*>(p.v) + head_off : nullptr;

  // This lane's query row (the column of the transposed score tile).
  const int qi = wave * 32 + (lane & 31);
  const bool wave_active = wave * 32 < M;
  const bool q_valid = qi < M;
  const int qtok = q0 + (rep ? (q_valid ? rowlist[qi] : 0) : qi);

  bf16x8 qf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    if (q_valid) {
      qf[ks] = *reinterpret_cast<const bf16x8*>(qg + (int64_t)qtok * p.sn + ks * 16 + g * 8);
    } else {
      qf[ks] = bf16x8{};
    }
  }

  // Key-block list of this row (no list: every key block, in order).
  const bool dense = p.row_ptr == nullptr;
  int beg = 0, nblk = p.nb;
  if (!dense) {
    beg = max(p.row_ptr[row], 0);
    const int64_t end = min((int64_t)p.row_ptr[row + 1], p.col_len);
    nblk = (int)max((int64_t)0, end - beg);
  }
  // Uniform across the wave: the skip-list reads become scalar loads.
  beg = __builtin_amdgcn_readfirstlane(beg);
  nblk = __builtin_amdgcn_readfirstlane(nblk);
  // The skip list is read-only for the kernel's lifetime: reading it through the
  // constant address space lets the (uniform) reads go to the scalar unit.
  const __attribute__((address_space(4))) int32_t* cidx =
      (const __attribute__((address_space(4))) int32_t*)p.col_idx;
  const __attribute__((address_space(4))) uint32_t* civ =
      (const __attribute__((address_space(4))) uint32_t*)p.ivs;
  // Runs: [beg, beg + nblk) indexes the row's runs; the blocks to visit are the
  // sum of their counts.  A cursor (run iv_j, offset iv_off) hands out the blocks
  // in order, one per call of step_key0 with s % SPB == 0 (its calls come in
  // increasing s).
  const int iv_end = beg + nblk;
  int iv_j = beg, iv_off = 0, iv_kb = -1;
  if (IV) {
    int tot = 0;
    for (int j = beg; j < iv_end; ++j) tot += (int)(civ[j] >> 16);
    nblk = tot;
  }
  const int nsteps = nblk * C::SPB;
  auto step_key0 = [&](int s) -> int {
    int kb;
    if (IV) {
      if (s % C::SPB == 0) {
        while (iv_j < iv_end && iv_off >= (int)(civ[iv_j] >> 16)) {
          ++iv_j;
          iv_off = 0;
        }
        iv_kb = iv_j < iv_end ? (int)(civ[iv_j] & 0xffffu) + iv_off : -1;
        ++iv_off;
      }
      kb = iv_kb;
    } else {
      kb = dense ? s / C::SPB : cidx[beg + s / C::SPB];
    }
    if (kb < 0 || kb >= p.nb) return -1;
    const int k0 = kb * B + (s % C::SPB) * C::KT;
    return k0 < p.n ? k0 : -1;
  };

  f32x16 oacc[PV ? C::DT : 1];
#pragma unroll
  for (int dt = 0; dt < (PV ? C::DT : 1); ++dt) oacc[dt] = f32x16{};
  float m_used = -INFINITY;  // reference maximum, base-2 units
  float l_part = 0.f;        // this lane's share of the exact row sum (LSE)
  float r_part = 0.f;        // this lane's share of the rounded-weight sum (O)

  // Even steps use buffers (k0s, v0s), odd steps (k1s, v1s).
  // BUF: tiles come by buffer loads with per-lane offsets fixed for the whole
  // item (byte offsets fit 32 bits); otherwise by global loads with the row
  // clamped to the sequence.
  constexpr int LPW = C::KT / (64 / (D / 8)) / C::NW;
  int voff[LPW];
  if (BUF) tile_lane_offsets<D, C::KT, C::NW>((int)(p.sn * 2), voff);
  const TileSrc ksrc = tile_src<D>(kg, p.n, p.sn), vsrc = tile_src<D>(vg, p.n, p.sn);
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  // A step with no key block (k0 < 0, uniform) stages nothing: its compute is skipped.
  auto load = [&](int k0, bfraw* kdst, bfraw* vdst) {
    if (k0 < 0) return;
    if (BUF) {
      load_tile_buf(ksrc, k0, voff, LPW, kdst + wv * LPW * 512);
      if (PV) load_tile_buf(vsrc, k0, voff, LPW, vdst + wv * LPW * 512);
    } else {
      load_tile<D, C::KT, C::NW>(kg, p.sn, p.n, k0, kdst);
      if (PV) load_tile<D, C::KT, C::NW>(vg, p.sn, p.n, k0, vdst);
    }
  };
  // Key offsets of the current step and the next one; the one after that is read
  // a full step ahead of its use, so the skip-list latency stays off the path.
  int k0_cur = nsteps > 0 ? step_key0(0) : -1;
  int k0_n1 = nsteps > 1 ? step_key0(1) : -1;
  if (nsteps > 0) load(k0_cur, k0s, v0s);

  auto step = [&](int s, const bfraw* kt, const bfraw* vt, bfraw* kn, bfraw* vn) {
    // This wave's loads of tile s are complete; after the barrier everyone's are,
    // and every wave is done reading the other buffers (step s - 1).
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int k0_next = k0_n1;
    if (s + 1 < nsteps) load(k0_next, kn, vn);
    k0_n1 = s + 2 < nsteps ? step_key0(s + 2) : -1;
    if (wave_active && k0_cur >= 0) {
      f32x16 sacc[C::ST];
      qk_step<D, C::KT>(kt, qf, sacc);
      if (k0_cur + C::KT > p.n) mask_ragged<C::ST>(sacc, p.n, k0_cur);
      bf16x8 pb[C::ST][2];
      softmax_step<C::ST, C::DT, PV, LSE>(sacc, p.c, m_used, l_part, r_part, oacc, pb);
      if (PV) pv_step<D, C::KT>(vt, pb, oacc);
    }
    k0_cur = k0_next;
  };
  int s = 0;
  for (; s + 1 < nsteps; s += 2) {
    step(s, k0s, v0s, k1s, v1s);
    step(s + 1, k1s, v1s, k0s, v0s);
  }
  if (s < nsteps) step(s, k0s, v0s, k1s, v1s);

  if (!wave_active) return;
  const float l_tot = l_part + other_half(l_part);
  const float r_tot = r_part + other_half(r_part);
  if (!q_valid) return;
  const float inv = r_tot > 0.f ? 1.f / r_tot : 0.f;
  const float lse_val = l_tot > 0.f ? (m_used + log2f(l_tot)) * kLn2 : -INFINITY;

  // Repetition heads: the anchor stands for the next stride-1 image rows of its frame.
  int n_follow = 0;
  if (rep && qtok >= p.n_prefix) {
    const int y = ((qtok - p.n_prefix) / p.gw) % p.gh;
    n_follow = min(p.anchor_stride - 1, p.gh - 1 - y);
  }

  if (PV && p.o) {
    bfraw* og = static_cast<bfraw*>(p.o) + head_off;
    const int n_copies = p.fuse_broadcast ? n_follow : 0;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(oacc[dt][r * 4 + e] * inv);
        const int d = dt * 32 + r * 8 + g * 4;
        for (int cp = 0; cp <= n_copies; ++cp) {
          *reinterpret_cast<bf16x4*>(og + (int64_t)(qtok + cp * p.gw) * p.sn + d) = w;
        }
      }
  }
  if ((LSE || !PV) && p.lse && g == 0) {
    float* lg = p.lse + ((int64_t)b * p.heads + h) * p.n;
    for (int cp = 0; cp <= n_follow; ++cp) lg[qtok + cp * p.gw] = lse_val;
  }
}

// One workgroup per item: item i = blockIdx.x is row work_order[i / batch] (or
// row i / batch when there is no order) and batch item i % batch.
template <int D, int B, bool PV, bool LSE, bool BUF, bool IV>
__global__ __launch_bounds__((Cfg<D, B>::NT), (min_wgs_per_cu<D, Cfg<D, B>::NT>())) void attn_bf16_kernel(AttnParams p) {
  using C = Cfg<D, B>;
  __shared__ __attribute__((aligned(16))) bfraw k0s[C::TILE], k1s[C::TILE];
  __shared__ __attribute__((aligned(16))) bfraw v0s[PV ? C::TILE : 8], v1s[PV ? C::TILE : 8];
  __shared__ int rowlist[B];
  __shared__ int wcnt[4];
  const int it = blockIdx.x / p.batch, b = blockIdx.x - it * p.batch;
  const int row = p.work_order ? p.work_order[it] : it;
  attn_item<D, B, PV, LSE, BUF, IV>(p, row, b, k0s, k1s, v0s, v1s, rowlist, wcnt);
}

// Block energy, sweep 2: E[qb, kb] = sum over the tile of exp(s_ij - lse_i), with
// lse cached by the dense sweep.  One workgroup per QPB consecutive query blocks of
// one (head, batch item): every key tile staged in LDS serves QPB * B query rows.
// Each wave sums its 32 rows' probabilities per key block in-lane, reduces across
// the wave, and the per-wave partials of each query block are added in wave order
// at the end, so the result is deterministic and independent of QPB.
template <int D, int B, int QPB, bool BUF>
__global__ __launch_bounds__((QPB * Cfg<D, B>::NT), 2) void energy_bf16_kernel(AttnParams p) {
  using C = Cfg<D, B>;
  constexpr int WPB = C::NW, NW = QPB * WPB, NT = NW * 64;  // waves per query block, per workgroup
  __shared__ __attribute__((aligned(16))) bfraw k0s[C::TILE], k1s[C::TILE];
  extern __shared__ float part[];  // [NW][nb]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5;
  const int item = blockIdx.x;
  const int it = item / p.batch, b = item - it * p.batch;
  const int nqg = (p.nb + QPB - 1) / QPB;
  const int h = it / nqg, qb0 = (it - h * nqg) * QPB;
  const int q0 = qb0 * B;
  const int M = min(QPB * B, p.n - q0);

  const int64_t head_off = (int64_t)b * p.sb + (int64_t)h * p.sh;
  const bfraw* qg = static_cast<const bfraw*>(p.q) + head_off;
  const bfraw* kg = static_cast<const bfraw*>(p.k) + head_off;
  const int qi = wave * 32 + (lane & 31);
  const bool wave_active = wave * 32 < M;
  const bool q_valid = qi < M;
  const int qtok = q0 + qi;

  bf16x8 qf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    qf[ks] = q_valid ? *reinterpret_cast<const bf16x8*>(qg + (int64_t)qtok * p.sn + ks * 16 + g * 8)
                     : bf16x8{};
  }
  // exp2(s*c - lse2) with lse2 = +inf gives 0: rows past the end add nothing.
  const float lse2 = q_valid ? p.lse[((int64_t)b * p.heads + h) * p.n + qtok] * kLog2e : INFINITY;

  const int nsteps = p.nb * C::SPB;
  auto step_key0 = [&](int s) -> int {
    const int k0 = (s / C::SPB) * B + (s % C::SPB) * C::KT;
    return k0 < p.n ? k0 : -1;
  };
  constexpr int LPW = C::KT / (64 / (D / 8)) / NW;
  int voff[LPW];
  if (BUF) tile_lane_offsets<D, C::KT, NW>((int)(p.sn * 2), voff);
  const TileSrc ksrc = tile_src<D>(kg, p.n, p.sn);
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  auto load = [&](int k0, bfraw* kdst) {
    if (k0 < 0) return;
    if (BUF) load_tile_buf(ksrc, k0, voff, LPW, kdst + wv * LPW * 512);
    else load_tile<D, C::KT, NW>(kg, p.sn, p.n, k0, kdst);
  };
  float esum = 0.f;
  int k0_cur = step_key0(0);
  load(k0_cur, k0s);
  auto step = [&](int s, const bfraw* kt, bfraw* kn) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int k0_next = -1;
    if (s + 1 < nsteps) {
      k0_next = step_key0(s + 1);
      load(k0_next, kn);
    }
    if (wave_active && k0_cur >= 0) {
      f32x16 sacc[C::ST];
      qk_step<D, C::KT>(kt, qf, sacc);
      if (k0_cur + C::KT > p.n) mask_ragged<C::ST>(sacc, p.n, k0_cur);
#pragma unroll
      for (int t = 0; t < C::ST; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) esum += __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][i], p.c, -lse2));
    }
    if (s % C::SPB == C::SPB - 1) {
      const float tot = wave_active ? wave_sum(esum) : 0.f;
      if (lane == 0) part[wave * p.nb + s / C::SPB] = tot;
      esum = 0.f;
    }
    k0_cur = k0_next;
  };
  int s = 0;
  for (; s + 1 < nsteps; s += 2) {
    step(s, k0s, k1s);
    step(s + 1, k1s, k0s);
  }
  if (s < nsteps) step(s, k0s, k1s);
  __syncthreads();
  for (int idx = tid; idx < QPB * p.nb; idx += NT) {
    const int j = idx / p.nb, kb = idx - j * p.nb;
    const int qb = qb0 + j;
    if (qb >= p.nb) continue;
    float e = 0.f;
    for (int w = j * WPB; w < (j + 1) * WPB; ++w) e += part[w * p.nb + kb];
    p.energy[(((int64_t)b * p.heads + h) * p.nb + qb) * p.nb + kb] = e;
  }
}

template <int D, int B>
hipError_t launch_attn_t(const AttnParams& p, bool with_pv, hipStream_t stream) {
  using C = Cfg<D, B>;
  const size_t lds = 0;  // static tile buffers
  const dim3 grid((unsigned)((int64_t)p.n_rows * p.batch)), block(C::NT);
  // Buffer loads take 32-bit byte offsets: every key row of a head must be
  // addressable with them.
  const bool buf = (int64_t)(p.n + C::KT) * p.sn * 2 < ((int64_t)1 << 31);
  void (*kern)(AttnParams);
  if (p.ivs) {  // interval skip list (with_pv only)
    if (p.lse) kern = buf ? attn_bf16_kernel<D, B, true, true, true, true> : attn_bf16_kernel<D, B, true, true, false, true>;
    else kern = buf ? attn_bf16_kernel<D, B, true, false, true, true> : attn_bf16_kernel<D, B, true, false, false, true>;
  } else if (!with_pv) {
    kern = buf ? attn_bf16_kernel<D, B, false, true, true, false> : attn_bf16_kernel<D, B, false, true, false, false>;
  } else if (p.lse) {
    kern = buf ? attn_bf16_kernel<D, B, true, true, true, false> : attn_bf16_kernel<D, B, true, true, false, false>;
  } else {
    kern = buf ? attn_bf16_kernel<D, B, true, false, true, false> : attn_bf16_kernel<D, B, true, false, false, false>;
  }
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  AttnParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel((const void*)kern, grid, block, args, lds, stream);
}

template <int D, int B, int QPB>
hipError_t launch_energy_q(const AttnParams& p, hipStream_t stream) {
  using C = Cfg<D, B>;
  const size_t lds = (size_t)QPB * C::NW * p.nb * sizeof(float);
  const int64_t nqg = (p.nb + QPB - 1) / QPB;
  const dim3 grid((unsigned)((int64_t)p.heads * nqg * p.batch)), block(QPB * C::NT);
  const bool buf = (int64_t)(p.n + C::KT) * p.sn * 2 < ((int64_t)1 << 31);
  auto kern = buf ? energy_bf16_kernel<D, B, QPB, true> : energy_bf16_kernel<D, B, QPB, false>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  AttnParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel((const void*)kern, grid, block, args, lds, stream);
}

template <int D, int B>
hipError_t launch_energy_t(const AttnParams& p, hipStream_t stream) {
  using C = Cfg<D, B>;
  constexpr int Q = energy_qpb<D, B>();
  // The per-wave partials grow with the waves: fall back to one query block per
  // workgroup when they would keep two workgroups from sharing a CU.
  const size_t lds = (size_t)Q * C::NW * p.nb * sizeof(float) + 2 * C::TILE * 2;
  if (Q > 1 && lds <= 64 * 1024) return launch_energy_q<D, B, Q>(p, stream);
  return launch_energy_q<D, B, 1>(p, stream);
}

}  // namespace

hipError_t launch_attn_bf16(const AttnParams& p, int head_dim, int block, bool with_pv, hipStream_t stream) {
#define CBA_CASE(D, B) \
  if (head_dim == D && block == B) return launch_attn_t<D, B>(p, with_pv, stream);
  CBA_CASE(64, 32) CBA_CASE(64, 64) CBA_CASE(64, 128)
  CBA_CASE(128, 32) CBA_CASE(128, 64) CBA_CASE(128, 128)
#undef CBA_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_energy_bf16(const AttnParams& p, int head_dim, int block, hipStream_t stream) {
#define CBA_CASE(D, B) \
  if (head_dim == D && block == B) return launch_energy_t<D, B>(p, stream);
  CBA_CASE(64, 32) CBA_CASE(64, 64) CBA_CASE(64, 128)
  CBA_CASE(128, 32) CBA_CASE(128, 64) CBA_CASE(128, 128)
#undef CBA_CASE
  return hipErrorInvalidValue;
}

}  // namespace cba
