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
template <int D, int KT, int NW>
__device__ inline void tile_lane_offsets(int row_bytes, int* voff) {
  constexpr int CPR = D / 8, RPI = 64 / CPR, LPW = KT / RPI / NW;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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

// PV: compute O (otherwise only the log-sum-exp, for the energy sweep).
// LSE: keep the exact fp32 row sum for the log-sum-exp output.
// O is normalised by the sum of the same bf16-rounded weights that multiply V, so
// rounding the weights perturbs a convex combination instead of scaling it.
}  // namespace dev
}  // namespace cba
