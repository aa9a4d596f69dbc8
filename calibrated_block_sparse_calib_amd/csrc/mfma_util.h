// Device helpers shared by the bf16 matrix-core kernels (gfx950).
#pragma once

#include "cba_internal.h"

namespace cba {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t bfraw;
#define LDS_AS __attribute__((address_space(3)))

// Tile configuration of the bf16 attention-shaped kernels: B query rows per work
// item in waves of 32 rows, K and V staged in KT-key steps.
template <int D, int B>
struct Cfg {
  static constexpr int NW = B / 32;              // waves, 32 query rows each
  static constexpr int NT = NW * 64;             // threads
  static constexpr int KT = B < 64 ? B : 64;     // keys per step
  static constexpr int SPB = B / KT;             // steps per key block
  static constexpr int TILE = KT * D;            // elements per K or V tile
  static constexpr int KS = D / 16;              // k-steps of the QK^T product
  static constexpr int DT = D / 32;              // 32-wide d tiles of O
  static constexpr int ST = KT / 32;             // 32-key score tiles per step
};

// Workgroups per CU that the bf16 kernels ask the compiler to fit (launch
// bounds).  Two for the tilings that reach two waves per SIMD; at head_dim 128
// the one-wave workgroups of blocks 64 and 32 cannot (their double-buffered
// tiles and registers allow one wave per SIMD), so they ask for one instead of
// a target the compiler would miss.
template <int D, int THREADS>
constexpr int min_wgs_per_cu() {
  return (D >= 128 && THREADS < 256) ? 1 : 2;
}

// Query blocks per energy workgroup: about 256 query rows (8 waves) share each K
// tile, as far as the tile splits over the waves.
template <int D, int B>
constexpr int energy_qpb() {
  using C = Cfg<D, B>;
  constexpr int max_waves = C::KT * D / 512;  // one 1 KB tile load per wave at least
  constexpr int waves = max_waves < 8 ? max_waves : 8;
  return waves / C::NW > 0 ? waves / C::NW : 1;
}

// The online softmax rescales its output only when a row maximum grows by more
// than this many units of log2: the weights stay below 2^8, which bf16 and the
// fp32 accumulators hold exactly as well as weights below 1.
constexpr float kLazyRescale = 8.0f;

// Maximum of the values held by lanes l and l ^ 32 (the same in both lanes).
__device__ inline float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Value held by lane (l ^ 32).
__device__ inline float other_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ inline f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// p points into LDS: the explicit address-space casts make the compiler emit
// ds_read instructions rather than flat loads.
__device__ inline bf16x8 lds_read8(const bfraw* p) {
  return *(const LDS_AS bf16x8*)(p);
}

__device__ inline i16x4 lds_read_tr(const bfraw* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(p));
}

// K and V tiles live in LDS unpadded, KT rows of D bf16, with the 16-byte chunks
// of row r XOR-swizzled by s(r).  The LDS serves 256 bytes (64 banks) at a time:
// a K fragment read puts 16 consecutive rows, same logical chunk, in one such
// group, and a transpose read of V puts 4 consecutive rows x 4 chunks in one.
// For 256-byte rows (D = 128), s(r) = 4*(r % 4) + (r / 4) % 4 gives 16 distinct
// chunks over any 16 consecutive rows and 4 distinct chunk quads over any 4
// aligned rows, so both reads are conflict-free; 128-byte rows (D = 64) use
// s(r) = 2*(r % 4) + (r / 4) % 2 over their 8 chunks.
template <int D>
__device__ inline int swz(int r) {
  return D >= 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 2 * (r & 3) + ((r >> 2) & 1);
}

// Element offset of (row r, column d) in a swizzled tile with D columns.
template <int D>
__device__ inline int tile_off(int r, int d) {
  return r * D + ((((d >> 3) ^ swz<D>(r)) << 3) | (d & 7));
}

// Fills a KT x D tile straight from global memory (global_load_lds_dwordx4: each
// lane's 16 bytes land at the instruction's LDS base + 16 * lane, no registers).
// NW waves split the tile; wave load j of a wave covers 1 KB = 64 / (D / 8) rows.
// Physical chunk i % (D/8) of row rr holds logical chunk (i % (D/8)) ^ swz(rr).
// Rows past the end of the sequence reread the last row, a valid input row: such
// keys are masked out of the scores and get zero weight.  Callers pass
// 0 <= k0 < n.
template <int D, int KT, int NW>
__device__ inline void load_tile(const bfraw* src, int64_t sn, int n, int k0, bfraw* tile) {
  constexpr int CPR = D / 8, RPI = 64 / CPR, LPW = KT / RPI / NW;
  static_assert(KT % (RPI * NW) == 0, "tile rows must split evenly over the waves");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kk0 = k0 < 0 ? 0 : k0;
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int blk = wave * LPW + j;
    const int rr = blk * RPI + lane / CPR;
    const int col = (lane % CPR) ^ swz<D>(rr);
    const int64_t off = (int64_t)min(kk0 + rr, n - 1) * sn + col * 8;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(src + off),
                                     (LDS_AS void*)(tile + blk * 512), 16, 0, 0);
  }
}

// Buffer-load variant of load_tile, for tiles addressed with 32-bit byte offsets:
// the lane offsets inside a tile are fixed (tile_lane_offsets, once per kernel)
// and the tile's first key only moves the buffer's base, a scalar computation, so
// a tile load costs no vector instructions.  The buffer of a tile starts at its
// first key row and ends at the last byte of the sequence: the range check
// applies to the lane offsets, so rows past the end read as zeros.  The resource
// is built here, in device-only code, because the host compilation also sees
// kernels and their lambdas and has no buffer-resource type.
// wave: this wave's index among the NW waves that share the tile.
template <int D, int KT, int NW>
__device__ inline void tile_lane_offsets(int row_bytes, int* voff, int wave = threadIdx.x >> 6) {
  constexpr int CPR = D / 8, RPI = 64 / CPR, LPW = KT / RPI / NW;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int rr = (wave * LPW + j) * RPI + lane / CPR;
    voff[j] = rr * row_bytes + ((lane % CPR) ^ swz<D>(rr)) * 16;
  }
}

// One head's rows of K or V as seen by the buffer loads: base, bytes per row and
// bytes from the base to the end of the last row's D values.
struct TileSrc {
  const bfraw* base;
  int row_bytes;
  int end_bytes;
};

template <int D>
__device__ inline TileSrc tile_src(const bfraw* base, int n, int64_t sn) {
  return TileSrc{base, (int)(sn * 2), (int)(((int64_t)(n - 1) * sn + D) * 2)};
}

// Stages the tile whose first key is k0 (0 <= k0 < n, uniform over the
// workgroup); lpw loads per wave, each of 64 lanes x 16 bytes, at dst.
__device__ __forceinline__ void load_tile_buf(const TileSrc& t, int k0, const int* voff, int lpw, bfraw* dst) {
  const int kk = __builtin_amdgcn_readfirstlane(k0);
  const char* b = reinterpret_cast<const char*>(t.base) + (int64_t)kk * t.row_bytes;
  const int nrec = t.end_bytes - kk * t.row_bytes;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(b), (short)0, nrec, 0x00020000);
#pragma unroll
  for (int j = 0; j < lpw; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(dst + j * 512), 16, voff[j], 0, 0, 0);
}

// Token rows of query block qb that this workgroup computes.  Normal heads: all
// rows.  Repetition heads: text rows and the anchor image rows (y % stride == 0).
// Writes the compacted in-block offsets to rowlist and returns their count.
template <int B, int NT>
__device__ int build_rowlist(const AttnParams& p, int q0, bool rep, int* rowlist, int* wcnt) {
  if (!rep) return min(B, p.n - q0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  bool flag = false;
  if (tid < B) {
    const int tok = q0 + tid;
    if (tok < p.n) {
      if (tok < p.n_prefix) {
        flag = true;
      } else {
        const int y = ((tok - p.n_prefix) / p.gw) % p.gh;
        flag = (y % p.anchor_stride) == 0;
      }
    }
  }
  const uint64_t bal = __ballot(flag);
  const int before = __popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0) wcnt[wave] = __popcll(bal);
  __syncthreads();
  int off = 0, total = 0;
  for (int w = 0; w < NT / 64; ++w) {
    off += (w < wave) ? wcnt[w] : 0;
    total += wcnt[w];
  }
  if (flag) rowlist[off + before] = tid;
  __syncthreads();
  return total;
}

// ---------------------------------------------------------------------------
// One key step of the attention-shaped kernels, shared by all of them so that
// their arithmetic is the same instruction for instruction.  Per wave: 32 query
// rows (lane l holds query l % 32 of the transposed score tile) against the KT
// keys of the step staged in LDS.
//
// Scores, transposed: S^T = K Q^T with v_mfma_f32_32x32x16_bf16.  sacc[t] holds
// keys t*32 .. t*32+31; element i of lane l is key t*32 + (i/4)*8 + (l/32)*4 + i%4
// for query l % 32.  The K fragments are read PF fragments ahead of the MFMA that
// consumes them, so LDS latency overlaps the matrix-core work.
template <int D, int KT>
__device__ __forceinline__ void qk_step(const bfraw* kt, const bf16x8* qf, f32x16* sacc) {
  constexpr int KS = D / 16, ST = KT / 32, NF = ST * KS, PF = 3;
  const int lane = threadIdx.x & 63, g = lane >> 5;
  auto kfrag = [&](int f) {
    return lds_read8(kt + tile_off<D>((f / KS) * 32 + (lane & 31), (f % KS) * 16 + g * 8));
  };
  bf16x8 kf[PF];
#pragma unroll
  for (int f = 0; f < PF; ++f) kf[f] = kfrag(f);
#pragma unroll
  for (int t = 0; t < ST; ++t) sacc[t] = f32x16{};
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const bf16x8 a = kf[f % PF];
    if (f + PF < NF) kf[f % PF] = kfrag(f + PF);
    sacc[f / KS] = mfma(a, qf[f % KS], sacc[f / KS]);
  }
}

// Keys at or past the end of the sequence (a ragged last step starting at key k0)
// take no part: their scores become -inf.  The empty asm keeps the caller's rare
// branch a real branch (the compiler would otherwise evaluate the compares and
// selects on every step).
template <int ST>
__device__ __forceinline__ void mask_ragged(f32x16* sacc, int n, int k0) {
  asm volatile("" ::: "memory");
  const int lim = n - k0 - (((threadIdx.x & 63) >> 5) * 4);
#pragma unroll
  for (int t = 0; t < ST; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (t * 32 + (i >> 2) * 8 + (i & 3) >= lim) sacc[t][i] = -INFINITY;
}

// Maximum of N values as a tree of three-input maxima (v_max3_f32): depth about
// log3 N instead of a chain of N / 2 dependent instructions.  Maxima are exact, so
// the grouping does not change the result.
template <int N>
__device__ __forceinline__ float tree_max(const float* v) {
  if constexpr (N == 1) {
    return v[0];
  } else if constexpr (N == 2) {
    return fmaxf(v[0], v[1]);
  } else {
    constexpr int A = (N + 2) / 3, Bn = (N + 1) / 3;
    return fmaxf(fmaxf(tree_max<A>(v), tree_max<Bn>(v + A)), tree_max<N - A - Bn>(v + A + Bn));
  }
}

// Maximum over this lane's scores of the step and the other half-wave's (the same
// query row).
template <int ST>
__device__ __forceinline__ float step_max(const f32x16* sacc) {
  float v[ST * 16];
#pragma unroll
  for (int t = 0; t < ST; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) v[t * 16 + i] = sacc[t][i];
  return halves_max(tree_max<ST * 16>(v));
}

// Online softmax of one step against the running reference m_used (base-2 units,
// scale c = softmax scale * log2 e): the reference rises, and O and the sums are
// rescaled, only when a row maximum grows by more than kLazyRescale, so most steps
// skip the rescale.  Writes the step's weights exp2(c*s - m_used) to pb as bf16
// (the B operand layout of pv_step) and adds them to the sums: r_part the rounded
// weights that multiply V (PV), l_part the fp32 weights (LSE, or the energy sweep
// without V).  O is normalised at the end by the rounded sum, so rounding the
// weights perturbs a convex combination instead of scaling it.
// EXT: one more running sum, x_part, rescaled and incremented like l_part (the
// one-pass energy keeps the current key block's share there).
template <int ST, int DT, bool PV, bool LSE, bool EXT = false>
__device__ __forceinline__ void softmax_step(const f32x16* sacc, float c, float& m_used, float& l_part,
                                             float& r_part, f32x16* oacc, bf16x8 (*pb)[2],
                                             float* x_part = nullptr) {
  const float mt = step_max<ST>(sacc) * c;
  if (__ballot(mt > m_used + kLazyRescale)) {
    asm volatile("" ::: "memory");  // rare: keep it a branch
    const float m_new = fmaxf(m_used, mt);
    const float alpha = __builtin_amdgcn_exp2f(m_used - m_new);
    l_part *= alpha;
    if (EXT) *x_part *= alpha;
    r_part *= alpha;
    if (PV) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
    }
    m_used = m_new;
  }
  float ps = 0.f;
#pragma unroll
  for (int t = 0; t < ST; ++t)
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[t][k2 * 8 + e], c, -m_used));
        if (LSE || !PV || EXT) ps += x;
        if (PV) pb[t][k2][e] = (__bf16)x;
      }
  l_part += ps;
  if (EXT) *x_part += ps;
  if (PV) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int t = 0; t < ST; ++t)
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 pair = {pb[t][k2][e], pb[t][k2][e + 1]};
          r_part = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, r_part, false);
        }
  }
}

// O^T += V^T P^T for one step: the V^T fragments come from the row-major V tile
// through the LDS transpose read, with the key order of each fragment matched to
// the order in which pb holds the weights.
template <int D, int KT>
__device__ __forceinline__ void pv_step(const bfraw* vt, const bf16x8 (*pb)[2], f32x16* oacc) {
  constexpr int ST = KT / 32, DT = D / 32;
  const int lane = threadIdx.x & 63, g = lane >> 5, G = lane >> 4, li = lane & 15;
#pragma unroll
  for (int t = 0; t < ST; ++t)
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const int krow = t * 32 + k2 * 16 + 4 * g + (li >> 2);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int dcol = dt * 32 + (G & 1) * 16 + 4 * (li & 3);
        const i16x4 lo = lds_read_tr(vt + tile_off<D>(krow, dcol));
        const i16x4 hi = lds_read_tr(vt + tile_off<D>(krow + 8, dcol));
        const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[dt] = mfma(va, pb[t][k2], oacc[dt]);
      }
    }
}

}  // namespace dev
}  // namespace cba
