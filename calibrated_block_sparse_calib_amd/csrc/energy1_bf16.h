// One-pass block energies of dense attention for gfx950 (bf16 operands on the
// matrix cores, fp32 accumulation): the scores of each (query, key) pair are
// computed once, the per-(row, key block) log-sums go to a caller workspace, and
// once each row's log-sum-exp is known the workgroup turns its rows' log-sums into
// the tile energies E[qb, kb] (the sum of the tile's attention probabilities of the
// CalibAtt calibration, zh S2.2A / fr S2B).  With V the same pass writes O.
//
// The per-step arithmetic is that of the dense attention kernel (attn_bf16.hip),
// step for step, so O and the log-sum-exp are that kernel's bits.  The kernel is
// instantiated in two translation units, without V (energy1_bf16.hip) and with V
// (energy1_o_bf16.hip), because the two measure fastest under different
// instruction-scheduling strategies (build.py).
#pragma once

#include <algorithm>

#include "cba_internal.h"
#include "mfma_util.h"

namespace cba {
namespace {

using namespace dev;

// Block energies in one pass (no separate LSE sweep).  One workgroup per QPB
// consecutive query blocks of one (head, batch item), as energy_bf16_kernel.  For
// each row and key block the pass keeps the block's partial sum of exp2(c*s - m)
// against the row's running reference m (rescaled with it) and, at the end of the
// block, stores its base-2 log-sum L = m + log2(partial) in the workspace.  After
// the last key block the row's log-sum-exp lse2 is known, and the workgroup
// reduces its own rows: E[qb, kb] = sum over the rows i of exp2(L_i(kb) - lse2_i),
// one wave per (query block, key block) pair at a time, in a fixed order, so the
// result does not depend on QPB.  Workspace layout: [batch, heads, nb (qb), nb (kb),
// B] floats, so the rows of one (qb, kb) are contiguous.
// PV: the pass also multiplies by V and writes O, step for step as attn_item's
// dense pass (same weights, same order), so O and the LSE are those of
// dense_attn_fwd bit for bit.
// Items run (batch item, head)-major: item = (b * heads + h) * nqg + query-block
// group, so a contiguous range of items owns a contiguous range of workspace rows
// (row = (b * heads + h) * nb + qb).  A launch covers items item0 + blockIdx.x and
// holds the workspace rows from ws_row0 on at ws, so a workspace smaller than the
// whole problem can serve it in several launches.
template <int D, int B, int QPB, bool PV, bool BUF>
__global__ __launch_bounds__((QPB * Cfg<D, B>::NT), (min_wgs_per_cu<D, QPB * Cfg<D, B>::NT>())) void energy1_bf16_kernel(AttnParams p, float* ws,
                                                                                int64_t item0, int64_t ws_row0) {
  using C = Cfg<D, B>;
  constexpr int NW = QPB * C::NW;  // waves per workgroup, 32 rows each
  __shared__ __attribute__((aligned(16))) bfraw k0s[C::TILE], k1s[C::TILE];
  __shared__ __attribute__((aligned(16))) bfraw v0s[PV ? C::TILE : 8], v1s[PV ? C::TILE : 8];
  __shared__ float lse2_s[QPB * B];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5;
  const int nqg = (p.nb + QPB - 1) / QPB;
  const int64_t item = item0 + blockIdx.x;
  const int bhi = (int)(item / nqg), qgrp = (int)(item - (int64_t)bhi * nqg);
  const int b = bhi / p.heads, h = bhi - b * p.heads;
  const int qb0 = qgrp * QPB;
  const int q0 = qb0 * B;
  const int M = min(QPB * B, p.n - q0);

  const int64_t head_off = (int64_t)b * p.sb + (int64_t)h * p.sh;
  const bfraw* qg = static_cast<const bfraw*>(p.q) + head_off;
  const bfraw* kg = static_cast<const bfraw*>(p.k) + head_off;
  const bfraw* vg = PV ? static_cast<const bfraw*>(p.v) + head_off : nullptr;
  const int qi = wave * 32 + (lane & 31);
  const bool wave_active = wave * 32 < M;
  const bool q_valid = qi < M;
  const int qtok = q0 + qi;
  const int64_t bh = bhi;
  // [kb][B] slice of this row's query block (only dereferenced for valid rows)
  float* wrow = ws + ((bh * p.nb + qb0 + qi / B - ws_row0) * (int64_t)p.nb) * B + qi % B;

  bf16x8 qf[C::KS];
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    qf[ks] = q_valid ? *reinterpret_cast<const bf16x8*>(qg + (int64_t)qtok * p.sn + ks * 16 + g * 8)
                     : bf16x8{};
  }

  const int nsteps = p.nb * C::SPB;
  auto step_key0 = [&](int s) -> int {
    const int k0 = (s / C::SPB) * B + (s % C::SPB) * C::KT;
    return k0 < p.n ? k0 : -1;
  };
  constexpr int LPW = C::KT / (64 / (D / 8)) / NW;
  int voff[LPW];
  if (BUF) tile_lane_offsets<D, C::KT, NW>((int)(p.sn * 2), voff);
  const TileSrc ksrc = tile_src<D>(kg, p.n, p.sn), vsrc = tile_src<D>(vg, p.n, p.sn);
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  auto load = [&](int k0, bfraw* kdst, bfraw* vdst) {
    if (k0 < 0) return;
    if (BUF) {
      load_tile_buf(ksrc, k0, voff, LPW, kdst + wv * LPW * 512);
      if (PV) load_tile_buf(vsrc, k0, voff, LPW, vdst + wv * LPW * 512);
    } else {
      load_tile<D, C::KT, NW>(kg, p.sn, p.n, k0, kdst);
      if (PV) load_tile<D, C::KT, NW>(vg, p.sn, p.n, k0, vdst);
    }
  };
  f32x16 oacc[PV ? C::DT : 1];
#pragma unroll
  for (int dt = 0; dt < (PV ? C::DT : 1); ++dt) oacc[dt] = f32x16{};
  float m_used = -INFINITY;  // reference maximum, base-2 units
  float l_part = 0.f;        // this lane's share of the row sum
  float b_part = 0.f;        // this lane's share of the current key block's sum
  float r_part = 0.f;        // this lane's share of the rounded-weight sum (O)
  int k0_cur = step_key0(0);
  load(k0_cur, k0s, v0s);
  auto step = [&](int s, const bfraw* kt, const bfraw* vt, bfraw* kn, bfraw* vn) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    int k0_next = -1;
    if (s + 1 < nsteps) {
      k0_next = step_key0(s + 1);
      load(k0_next, kn, vn);
    }
    if (wave_active && k0_cur >= 0) {
      f32x16 sacc[C::ST];
      qk_step<D, C::KT>(kt, qf, sacc);
      if (k0_cur + C::KT > p.n) mask_ragged<C::ST>(sacc, p.n, k0_cur);
      bf16x8 pb[C::ST][2];
      softmax_step<C::ST, C::DT, PV, true, true>(sacc, p.c, m_used, l_part, r_part, oacc, pb, &b_part);
      if (PV) pv_step<D, C::KT>(vt, pb, oacc);
    }
    if (s % C::SPB == C::SPB - 1) {
      // End of key block s / SPB: its base-2 log-sum for this lane's row.
      const float bt = b_part + other_half(b_part);
      if (q_valid && g == 0) wrow[(int64_t)(s / C::SPB) * B] = m_used + __builtin_log2f(bt);
      b_part = 0.f;
    }
    k0_cur = k0_next;
  };
  int s = 0;
  for (; s + 1 < nsteps; s += 2) {
    step(s, k0s, v0s, k1s, v1s);
    step(s + 1, k1s, v1s, k0s, v0s);
  }
  if (s < nsteps) step(s, k0s, v0s, k1s, v1s);

  // Row log-sum-exp: LSE output (natural log) and, for the reduction, base 2.
  if (wave_active) {
    const float l_tot = l_part + other_half(l_part);
    const float lse2 = l_tot > 0.f ? m_used + log2f(l_tot) : -INFINITY;
    if (g == 0) {
      lse2_s[qi] = q_valid ? lse2 : INFINITY;  // rows past the end add nothing
      if (q_valid) p.lse[bh * p.n + qtok] = lse2 * kLn2;
    }
    if (PV) {
      const float r_tot = r_part + other_half(r_part);
      const float inv = r_tot > 0.f ? 1.f / r_tot : 0.f;
      if (q_valid) {
        bfraw* og = static_cast<bfraw*>(p.o) + head_off + (int64_t)qtok * p.sn;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            bf16x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) w[e] = (__bf16)(oacc[dt][r * 4 + e] * inv);
            *reinterpret_cast<bf16x4*>(og + dt * 32 + r * 8 + g * 4) = w;
          }
      }
    }
  } else if (lane < 32) {
    lse2_s[qi] = INFINITY;
  }
  __syncthreads();  // workspace writes and lse2_s visible to the workgroup
  // E[qb0 + j, kb]: wave w reduces pairs (j, kb) = w, w + NW, ... in row-major
  // order; lane l takes rows l, l + 64 of the query block.
  for (int idx = wave; idx < QPB * p.nb; idx += NW) {
    const int j = idx / p.nb, kb = idx - j * p.nb;
    const int Mj = M - j * B;  // valid rows of query block qb0 + j
    if (Mj <= 0) break;        // uniform over the wave; later pairs have larger j
    const float* L = ws + ((bh * p.nb + qb0 + j - ws_row0) * (int64_t)p.nb + kb) * B;
    float e = 0.f;
#pragma unroll
    for (int r = lane; r < B; r += 64)
      if (r < Mj) e += __builtin_amdgcn_exp2f(L[r] - lse2_s[j * B + r]);
    e = wave_sum(e);
    if (lane == 0) p.energy[(bh * p.nb + qb0 + j) * p.nb + kb] = e;
  }
}

// Query blocks per one-pass workgroup: as for the two-sweep energy (about 256 rows).
template <int D, int B>
constexpr int energy1_qpb() {
  return energy_qpb<D, B>();
}

// Launch with Q query blocks per workgroup (with V, Q = 1 as in the dense pass).
// ws_bytes < 0: ws holds the whole problem's workspace, one launch.  Otherwise ws
// holds ws_bytes and the items go in consecutive launches, each over the longest
// run of items whose workspace rows fit.
template <int D, int B, int Q, bool PV>
hipError_t launch_energy1_q(const AttnParams& p, float* ws, int64_t ws_bytes, hipStream_t stream) {
  using C = Cfg<D, B>;
  const int64_t nqg = (p.nb + Q - 1) / Q;
  const int64_t n_items = (int64_t)p.heads * p.batch * nqg;
  const dim3 block(Q * C::NT);
  const bool buf = (int64_t)(p.n + C::KT) * p.sn * 2 < ((int64_t)1 << 31);
  auto kern = buf ? energy1_bf16_kernel<D, B, Q, PV, true> : energy1_bf16_kernel<D, B, Q, PV, false>;
  AttnParams arg = p;
  float* w = ws;
  const int64_t row_bytes = (int64_t)p.nb * B * (int64_t)sizeof(float);
  // First workspace row of item i and one past its last.
  auto row_lo = [&](int64_t i) { return (i / nqg) * p.nb + (i % nqg) * Q; };
  auto row_hi = [&](int64_t i) { return (i / nqg) * p.nb + std::min<int64_t>((i % nqg) * Q + Q, p.nb); };
  const int64_t max_rows = ws_bytes < 0 ? row_hi(n_items - 1) : ws_bytes / row_bytes;
  for (int64_t i0 = 0; i0 < n_items;) {
    int64_t i1 = n_items;
    int64_t r0 = row_lo(i0);
    if (ws_bytes >= 0) {
      // largest i1 with row_hi(i1 - 1) - r0 <= max_rows (row_hi grows with i)
      int64_t lo = i0, hi = n_items;  // row_hi(lo) - r0 <= max_rows is checked below
      if (row_hi(i0) - r0 > max_rows) return hipErrorInvalidValue;
      while (hi - lo > 1) {
        const int64_t mid = lo + (hi - lo) / 2;
        if (row_hi(mid) - r0 <= max_rows) lo = mid;
        else hi = mid;
      }
      i1 = lo + 1;
    } else {
      r0 = 0;
    }
    const dim3 grid((unsigned)(i1 - i0));
    int64_t it0 = i0, wr0 = r0;
    void* args[] = {&arg, &w, &it0, &wr0};
    hipError_t e = hipLaunchKernel((const void*)kern, grid, block, args, 0, stream);
    if (e != hipSuccess) return e;
    i0 = i1;
  }
  return hipSuccess;
}

}  // namespace
}  // namespace cba
