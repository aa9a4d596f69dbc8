// Integer and ordering kernels: energy-threshold block selection with cross-draw
// voting, the CSR skip list with its longest-first work order, and the anchor-row
// broadcast copy.
#include "cba_internal.h"

namespace cba {
namespace {

// ---------------------------------------------------------------- selection
//
// One workgroup per mask row (h, qb).  For every draw the row's energies are
// sorted in LDS by the 64-bit key (energy descending, index ascending) with a
// bitonic network; the sorted energies are promoted to fp64 and one thread adds
// them one at a time in sorted order (so the running sums are the same bits as a
// sequential fp64 accumulation in that order); the first position reaching
// tau * total is found in parallel and the blocks before it get a vote.
constexpr int kSelThreads = 256;

__device__ inline uint32_t sortable_desc(float f) {
  // Map so that ascending order of the result is descending order of f
  // (finite values; -0 is treated as +0).
  uint32_t u = __float_as_uint(f == 0.f ? 0.f : f);
  const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~asc;
}

__global__ __launch_bounds__(kSelThreads) void select_kernel(const float* energy, int n_draws, int heads,
                                                             int nb, TauTable taus, double rho, int force_diag,
                                                             int n_prefix_blocks, uint8_t* mask,
                                                             int32_t* votes_out) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  int p2 = 1;
  while (p2 < nb) p2 <<= 1;
  uint64_t* keys = reinterpret_cast<uint64_t*>(smem);    // [p2]
  double* run = reinterpret_cast<double*>(keys + p2);     // [nb]
  float* vals = reinterpret_cast<float*>(run + nb);       // [nb]
  int* vote = reinterpret_cast<int*>(vals + nb);          // [nb]
  __shared__ int kstar;

  const int tid = threadIdx.x;
  const int row = blockIdx.x;
  const int h = row / nb, qb = row - h * nb;
  const double tau = taus.per_head ? taus.t[h] : taus.t[0];
  for (int j = tid; j < nb; j += kSelThreads) vote[j] = (tau >= 1.0) ? n_draws : 0;

  if (tau < 1.0) {
    for (int d = 0; d < n_draws; ++d) {
      const float* e = energy + (((int64_t)d * heads + h) * nb + qb) * nb;
      for (int j = tid; j < p2; j += kSelThreads) {
        if (j < nb) {
          const float f = e[j];
          vals[j] = f;
          keys[j] = ((uint64_t)sortable_desc(f) << 32) | (uint32_t)j;
        } else {
          keys[j] = ~0ull;
        }
      }
      __syncthreads();
      for (int k = 2; k <= p2; k <<= 1) {
        for (int jj = k >> 1; jj > 0; jj >>= 1) {
          for (int i = tid; i < p2; i += kSelThreads) {
            const int ixj = i ^ jj;
            if (ixj > i) {
              const uint64_t a = keys[i], c = keys[ixj];
              const bool up = (i & k) == 0;
              if ((a > c) == up) {
                keys[i] = c;
                keys[ixj] = a;
              }
            }
          }
          __syncthreads();
        }
      }
      for (int k = tid; k < nb; k += kSelThreads) run[k] = (double)vals[keys[k] & 0xffffffffu];
      __syncthreads();
      if (tid == 0) {
        double s = 0.0;
        for (int k = 0; k < nb; ++k) {
          s += run[k];
          run[k] = s;
        }
        kstar = nb - 1;
      }
      __syncthreads();
      const double target = tau * run[nb - 1];
      for (int k = tid; k < nb; k += kSelThreads)
        if (run[k] >= target) atomicMin(&kstar, k);
      __syncthreads();
      const int ks = kstar;
      for (int k = tid; k <= ks; k += kSelThreads) vote[keys[k] & 0xffffffffu] += 1;
      __syncthreads();
    }
  }
  const double need = rho * (double)n_draws;
  uint8_t* mrow = mask + (int64_t)row * nb;
  for (int j = tid; j < nb; j += kSelThreads) {
    bool keep = (double)vote[j] > need;
    if (force_diag && j == qb) keep = true;
    if (qb < n_prefix_blocks || j < n_prefix_blocks) keep = true;
    mrow[j] = keep ? 1 : 0;
    if (votes_out) votes_out[(int64_t)row * nb + j] = vote[j];
  }
}

// ---------------------------------------------------------------- CSR
//
// count: one wave per row writes its kept count to row_ptr[r + 1];
// scan:  one workgroup turns the counts into running totals in place;
// fill:  one wave per row writes its kept indices in ascending order;
// order: one workgroup per count value c places the rows with count c, in row
//        order, after all rows with a larger count.
constexpr int kWaves = 4;

__global__ __launch_bounds__(64 * kWaves) void csr_count_kernel(const uint8_t* mask, int n_rows, int nkb,
                                                               int32_t* row_ptr) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (blockIdx.x == 0 && threadIdx.x == 0) row_ptr[0] = 0;
  if (row >= n_rows) return;
  const uint8_t* m = mask + (int64_t)row * nkb;
  int cnt = 0;
  for (int j0 = 0; j0 < nkb; j0 += 64) {
    const int j = j0 + lane;
    cnt += __popcll(__ballot(j < nkb && m[j] != 0));
  }
  if (lane == 0) row_ptr[row + 1] = cnt;
}

constexpr int kScanThreads = 1024;
constexpr int kScanPer = 16;  // counts per thread per pass: 16 K rows per pass
constexpr int kScanChunk = kScanThreads * kScanPer;

// Padded LDS index: a thread's run of kScanPer consecutive counts then spans
// distinct banks.
__device__ inline int scan_slot(int i) { return i + (i >> 4); }

// In-place inclusive scan of row_ptr[1 .. n_rows] (the per-row counts) by one
// workgroup.  Each pass stages 16 K counts in LDS with coalesced loads; every
// thread sums its own run of kScanPer counts, the workgroup scans the run totals
// (wave scans, then the wave totals), each thread writes its run's prefixes back
// to LDS, and the pass ends with coalesced stores.
__global__ __launch_bounds__(kScanThreads) void csr_scan_kernel(int n_rows, int32_t* row_ptr) {
  __shared__ int buf[kScanChunk + kScanChunk / 16];
  __shared__ int wsum[kScanThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int carry = 0;
  for (int base = 0; base < n_rows; base += kScanChunk) {
    const int len = min(kScanChunk, n_rows - base);
    for (int i = tid; i < kScanChunk; i += kScanThreads) buf[scan_slot(i)] = i < len ? row_ptr[base + i + 1] : 0;
    __syncthreads();
    int v[kScanPer];
    int run = 0;
#pragma unroll
    for (int i = 0; i < kScanPer; ++i) {
      v[i] = buf[scan_slot(tid * kScanPer + i)];
      run += v[i];
    }
    int x = run;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int before = carry, total = carry;
    for (int w = 0; w < kScanThreads / 64; ++w) {
      before += (w < wave) ? wsum[w] : 0;
      total += wsum[w];
    }
    int acc = before + x - run;  // exclusive prefix of this thread's run
#pragma unroll
    for (int i = 0; i < kScanPer; ++i) {
      acc += v[i];
      buf[scan_slot(tid * kScanPer + i)] = acc;
    }
    __syncthreads();
    for (int i = tid; i < len; i += kScanThreads) row_ptr[base + i + 1] = buf[scan_slot(i)];
    carry = total;
    __syncthreads();
  }
}

__global__ __launch_bounds__(64 * kWaves) void csr_fill_kernel(const uint8_t* mask, int n_rows, int nkb,
                                                              const int32_t* row_ptr, int32_t* col_idx,
                                                              int64_t capacity) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= n_rows) return;
  const uint8_t* m = mask + (int64_t)row * nkb;
  int64_t pos0 = row_ptr[row];
  for (int j0 = 0; j0 < nkb; j0 += 64) {
    const int j = j0 + lane;
    const bool f = j < nkb && m[j] != 0;
    const uint64_t bal = __ballot(f);
    const int64_t pos = pos0 + __popcll(bal & ((1ull << lane) - 1ull));
    if (f && pos < capacity) col_idx[pos] = j;
    pos0 += __popcll(bal);
  }
}

constexpr int kOrderThreads = 256;

// Longest-first order (heavy_first = 0): workgroup c places the rows with kept
// count c, in row order, after all rows with a larger count.  Heavy-first order
// (heavy_first = 1): only counts above thr = factor * mean are placed that way;
// one more workgroup (c = gridDim.x - 1) places every other row, in row order,
// after all the heavy rows.
__global__ __launch_bounds__(kOrderThreads) void csr_order_kernel(int n_rows, const int32_t* row_ptr,
                                                                  int32_t* work_order, int heavy_first,
                                                                  double factor) {
  __shared__ int wcnt[kOrderThreads / 64];
  __shared__ int total_s;
  const int c = blockIdx.x;  // the kept count handled by this workgroup
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const double thr = heavy_first ? factor * ((double)row_ptr[n_rows] / (double)n_rows) : -1.0;
  const bool light_group = heavy_first && c == (int)gridDim.x - 1;
  if (heavy_first && !light_group && (double)c <= thr) return;  // light count: placed by the last group
  // Rows placed before this group's: a larger count, or (light group) every heavy row.
  int gt = 0;
  for (int r = tid; r < n_rows; r += kOrderThreads) {
    const int cnt = row_ptr[r + 1] - row_ptr[r];
    gt += light_group ? ((double)cnt > thr) : (cnt > c);
  }
  for (int off = 32; off >= 1; off >>= 1) gt += __shfl_xor(gt, off, 64);
  if (lane == 0) wcnt[wave] = gt;
  __syncthreads();
  if (tid == 0) {
    int s = 0;
    for (int w = 0; w < kOrderThreads / 64; ++w) s += wcnt[w];
    total_s = s;
  }
  __syncthreads();
  int pos = total_s;
  __syncthreads();
  for (int base = 0; base < n_rows; base += kOrderThreads) {
    const int r = base + tid;
    const int cnt = r < n_rows ? row_ptr[r + 1] - row_ptr[r] : 0;
    const bool f = r < n_rows && (light_group ? (double)cnt <= thr : cnt == c);
    const uint64_t bal = __ballot(f);
    if (lane == 0) wcnt[wave] = __popcll(bal);
    __syncthreads();
    int before = pos, chunk = 0;
    for (int w = 0; w < kOrderThreads / 64; ++w) {
      before += (w < wave) ? wcnt[w] : 0;
      chunk += wcnt[w];
    }
    if (f) work_order[before + __popcll(bal & ((1ull << lane) - 1ull))] = r;
    pos += chunk;
    __syncthreads();
  }
}

// ---------------------------------------------------------------- intervals
//
// Runs of consecutive kept blocks, one packed word per run: first block in the
// low 16 bits, block count in the high 16 bits.  One wave per row walks the row
// 64 blocks at a time with ballots.  In a chunk with kept bits K (bit l = block
// j0 + l), a run starts at l when K has l and not l - 1 (the bit before the chunk
// comes from the previous chunk), and ends at l when K has l and not l + 1 (the bit
// after the chunk comes from the next chunk).  A run ending at l began at the
// highest start at or below l in the chunk, or, if there is none, in an earlier
// chunk (the run still open when the chunk began).
// count: runs per row into iv_ptr[r + 1]; the CSR scan then makes them offsets;
// fill:  each end lane writes its run at its rank among the row's runs.

__device__ inline uint64_t chunk_bits(const uint8_t* m, int nkb, int j0) {
  const int j = j0 + (threadIdx.x & 63);
  return __ballot(j < nkb && m[j] != 0);
}

__global__ __launch_bounds__(64 * kWaves) void iv_count_kernel(const uint8_t* mask, int n_rows, int nkb,
                                                              int32_t* iv_ptr) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (blockIdx.x == 0 && threadIdx.x == 0) iv_ptr[0] = 0;
  if (row >= n_rows) return;
  const uint8_t* m = mask + (int64_t)row * nkb;
  uint64_t carry = 0;
  int cnt = 0;
  for (int j0 = 0; j0 < nkb; j0 += 64) {
    const uint64_t k = chunk_bits(m, nkb, j0);
    cnt += __popcll(k & ~((k << 1) | carry));
    carry = k >> 63;
  }
  if (lane == 0) iv_ptr[row + 1] = cnt;
}

__global__ __launch_bounds__(64 * kWaves) void iv_fill_kernel(const uint8_t* mask, int n_rows, int nkb,
                                                             const int32_t* iv_ptr, uint32_t* ivs,
                                                             int64_t capacity) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= n_rows) return;
  const uint8_t* m = mask + (int64_t)row * nkb;
  int64_t pos0 = iv_ptr[row];
  uint64_t carry = 0;
  int open_first = 0;  // first block of the run open at the start of the chunk
  uint64_t k = chunk_bits(m, nkb, 0);
  for (int j0 = 0; j0 < nkb; j0 += 64) {
    const uint64_t k_next = j0 + 64 < nkb ? chunk_bits(m, nkb, j0 + 64) : 0;
    const uint64_t starts = k & ~((k << 1) | carry);
    const uint64_t ends = k & ~((k >> 1) | (k_next << 63));
    if ((ends >> lane) & 1) {
      const uint64_t s_le = starts & ((2ull << lane) - 1ull);  // starts at or below this lane
      const int first = s_le ? j0 + 63 - __clzll(s_le) : open_first;
      const int64_t pos = pos0 + __popcll(ends & ((1ull << lane) - 1ull));
      if (pos < capacity) ivs[pos] = (uint32_t)first | ((uint32_t)(j0 + lane - first + 1) << 16);
    }
    pos0 += __popcll(ends);
    if (starts) open_first = j0 + 63 - __clzll(starts);  // only used while a run stays open
    carry = k >> 63;
    k = k_next;
  }
}

// ---------------------------------------------------------------- broadcast
//
// One workgroup per (image row (f, y), batch * head).  Follower rows of repetition
// heads copy the W tokens of their anchor row, 16 bytes per thread per step.
__global__ __launch_bounds__(256) void broadcast_kernel(AttnParams p, int row_bytes, int elem_bytes) {
  const int bh = blockIdx.y;
  const int b = bh / p.heads, h = bh - b * p.heads;
  if (!rep_head(p, h)) return;
  const int fr = blockIdx.x;
  const int f = fr / p.gh, y = fr - f * p.gh;
  const int s = p.anchor_stride;
  if (y % s == 0) return;
  const int ya = (y / s) * s;
  char* base = static_cast<char*>(p.o) + ((int64_t)b * p.sb + (int64_t)h * p.sh) * elem_bytes;
  const int64_t src_tok = p.n_prefix + ((int64_t)f * p.gh + ya) * p.gw;
  const int64_t dst_tok = p.n_prefix + ((int64_t)f * p.gh + y) * p.gw;
  const int chunks = row_bytes / 16;
  const int64_t tok_bytes = p.sn * elem_bytes;
  for (int idx = threadIdx.x; idx < p.gw * chunks; idx += 256) {
    const int t = idx / chunks, c = idx - t * chunks;
    const uint4 v = *reinterpret_cast<const uint4*>(base + (src_tok + t) * tok_bytes + c * 16);
    *reinterpret_cast<uint4*>(base + (dst_tok + t) * tok_bytes + c * 16) = v;
  }
}

}  // namespace

hipError_t launch_select(const float* energy, int n_draws, int heads, int nb, const TauTable& taus, double rho,
                         int force_diag, int n_prefix_blocks, uint8_t* mask, int32_t* votes,
                         hipStream_t stream) {
  int p2 = 1;
  while (p2 < nb) p2 <<= 1;
  const size_t lds = (size_t)p2 * 8 + (size_t)nb * (8 + 4 + 4);
  hipError_t e = hipFuncSetAttribute((const void*)select_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)((int64_t)heads * nb)), dim3(kSelThreads), lds, stream,
                     energy, n_draws, heads, nb, taus, rho, force_diag, n_prefix_blocks, mask, votes);
  return hipGetLastError();
}

hipError_t launch_csr(const uint8_t* mask, int n_rows, int nkb, int32_t* row_ptr, int32_t* col_idx,
                      int64_t capacity, int32_t* work_order, hipStream_t stream) {
  const dim3 rows_grid((unsigned)((n_rows + kWaves - 1) / kWaves));
  hipLaunchKernelGGL(csr_count_kernel, rows_grid, dim3(64 * kWaves), 0, stream, mask, n_rows, nkb, row_ptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(csr_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, n_rows, row_ptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (col_idx) {
    hipLaunchKernelGGL(csr_fill_kernel, rows_grid, dim3(64 * kWaves), 0, stream, mask, n_rows, nkb,
                       (const int32_t*)row_ptr, col_idx, capacity);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (work_order) {
    hipLaunchKernelGGL(csr_order_kernel, dim3((unsigned)(nkb + 1)), dim3(kOrderThreads), 0, stream, n_rows,
                       (const int32_t*)row_ptr, work_order, 0, 0.0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_heavy_order(const int32_t* row_ptr, int n_rows, int nkb, double factor, int32_t* work_order,
                              hipStream_t stream) {
  hipLaunchKernelGGL(csr_order_kernel, dim3((unsigned)(nkb + 2)), dim3(kOrderThreads), 0, stream, n_rows, row_ptr,
                     work_order, 1, factor);
  return hipGetLastError();
}

hipError_t launch_intervals(const uint8_t* mask, int n_rows, int nkb, int32_t* iv_ptr, uint32_t* ivs,
                            int64_t capacity, hipStream_t stream) {
  const dim3 rows_grid((unsigned)((n_rows + kWaves - 1) / kWaves));
  hipLaunchKernelGGL(iv_count_kernel, rows_grid, dim3(64 * kWaves), 0, stream, mask, n_rows, nkb, iv_ptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(csr_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, n_rows, iv_ptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ivs) {
    hipLaunchKernelGGL(iv_fill_kernel, rows_grid, dim3(64 * kWaves), 0, stream, mask, n_rows, nkb,
                       (const int32_t*)iv_ptr, ivs, capacity);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_broadcast(const AttnParams& p, int head_dim, int elem_bytes, hipStream_t stream) {
  const dim3 grid((unsigned)(p.gf * p.gh), (unsigned)(p.batch * p.heads));
  hipLaunchKernelGGL(broadcast_kernel, grid, dim3(256), 0, stream, p, head_dim * elem_bytes, elem_bytes);
  return hipGetLastError();
}

}  // namespace cba
