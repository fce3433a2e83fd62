// sort.hip -- groups edges given in any order by destination node (a counting
// sort on the GPU) so that the dst-segmented convolution, which needs CSR row
// pointers, can run on them instead of the fp32-atomic scatter.
//
// eqtp_sort_edges needs no scratch memory: the row-pointer output doubles as
// the counter array.
//   1. row_ptr[0..N-1] = 0, then row_ptr[d] += 1 per edge (histogram);
//   2. one workgroup turns it in place into inclusive sums (row ends) and sets
//      row_ptr[N] = E;
//   3. every edge takes slot = atomicSub(&row_ptr[d], 1) - 1, which fills row
//      d from its end backwards and leaves row_ptr[d] at the row's start; the
//      edge's index (and, for eqtp_sort_edges, its vector and source) goes to
//      the slot.  The order inside a row follows the atomics.
// The convolution over edges in any order (eqtp_conv_fused_ws) has a
// workspace, and groups the edges with a stable LSD radix sort of the pairs
// (destination, edge index) instead: every row then holds its edges in input
// order, so the grouping and the convolution after it do not depend on any
// atomic's order.  Per pass over a digit of at most 9 bits:
//   * upsweep: each workgroup counts its tile's digits in LDS;
//   * the counts, digit-major over the tiles, are scanned per digit (one
//     workgroup each), then the digit totals;
//   * downsweep: each workgroup walks its tile (up to 16 rounds of 256 items;
//     fewer for small E, so that there are enough tiles to fill the chip)
//     again in input order; an item's place is its digit's offset for the tile,
//     plus the items with the same digit in the tile's earlier rounds and
//     waves, plus its rank among the lanes of its wave with the same digit
//     (found with one ballot per digit bit).
// Row pointers are then read off the sorted keys (each boundary written once)
// and vec and src are gathered in the sorted order.
#include "eqtp_device.hpp"
#include "eqtp_kernels.hpp"

namespace eqtp {

constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(256) void zero_i32_kernel(int* __restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

__global__ __launch_bounds__(256) void dst_histogram_kernel(const int* __restrict__ dst, int E, int N,
                                                            int* __restrict__ counts) {
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < E; e += gridDim.x * blockDim.x)
    atomicAdd(&counts[clamp_index(dst[e], N)], 1);
}

// In-place inclusive prefix sum of a[0..N-1] by one workgroup, then a[N] = E.
// The array is walked in tiles of kScanThreads * kScanItems entries: a tile is
// read coalesced into LDS (padded by one word per kScanItems so that the
// per-thread reads below do not collide in banks), each thread scans its
// kScanItems consecutive entries, the per-thread totals are scanned with
// shuffles inside each wave and through LDS across the waves, the tile is
// rewritten in LDS and stored coalesced; a running carry links the tiles.
constexpr int kScanItems = 8;
constexpr int kScanTile = kScanThreads * kScanItems;
__device__ __forceinline__ int scan_pad(int i) { return i + i / kScanItems; }

__global__ __launch_bounds__(kScanThreads) void inclusive_scan_kernel(int* __restrict__ a, int N, int E) {
  __shared__ int tile[kScanTile + kScanTile / kScanItems];
  __shared__ int wave_tot[kScanThreads / 64];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  int carry = 0;
  for (int base = 0; base < N; base += kScanTile) {
#pragma unroll
    for (int j = 0; j < kScanItems; ++j) {
      const int i = base + j * kScanThreads + t;
      tile[scan_pad(j * kScanThreads + t)] = i < N ? a[i] : 0;
    }
    __syncthreads();
    int v[kScanItems];
    int sum = 0;
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) {
      sum += tile[scan_pad(t * kScanItems + k)];
      v[k] = sum;
    }
    int incl = sum;  // inclusive scan of the per-thread totals inside the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int u = __shfl_up(incl, off, 64);
      if (lane >= off) incl += u;
    }
    if (lane == 63) wave_tot[wv] = incl;
    __syncthreads();
    int before = carry, all = 0;
#pragma unroll
    for (int w = 0; w < kScanThreads / 64; ++w) {
      const int s = wave_tot[w];
      before += w < wv ? s : 0;
      all += s;
    }
    const int off = before + incl - sum;  // exclusive prefix of this thread's entries
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) tile[scan_pad(t * kScanItems + k)] = off + v[k];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kScanItems; ++j) {
      const int i = base + j * kScanThreads + t;
      if (i < N) a[i] = tile[scan_pad(j * kScanThreads + t)];
    }
    carry += all;
    __syncthreads();  // the next tile overwrites tile[] and wave_tot[]
  }
  if (t == 0) a[N] = E;
}

__global__ __launch_bounds__(256) void scatter_by_dst_kernel(const int* __restrict__ dst, const float* __restrict__ vec,
                                                             const int* __restrict__ src, int E, int N,
                                                             int* __restrict__ ends, int* __restrict__ perm,
                                                             float* __restrict__ vec_out, int* __restrict__ src_out) {
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < E; e += gridDim.x * blockDim.x) {
    const int d = clamp_index(dst[e], N);
    const int slot = atomicSub(&ends[d], 1) - 1;
    perm[slot] = e;
    if (vec_out != nullptr) {
      vec_out[3 * (size_t)slot] = vec[3 * (size_t)e];
      vec_out[3 * (size_t)slot + 1] = vec[3 * (size_t)e + 1];
      vec_out[3 * (size_t)slot + 2] = vec[3 * (size_t)e + 2];
    }
    if (src_out != nullptr) src_out[slot] = src[e];
  }
}

// rows[e] = the row of CSR position e (one thread per row, grid-stride)
__global__ __launch_bounds__(256) void edge_rows_kernel(const int* __restrict__ row_ptr, int N, int E,
                                                        int* __restrict__ rows) {
  for (int r = blockIdx.x * blockDim.x + threadIdx.x; r < N; r += gridDim.x * blockDim.x) {
    const int b = min(max(row_ptr[r], 0), E);
    const int e = min(max(row_ptr[r + 1], b), E);
    for (int i = b; i < e; ++i) rows[i] = r;
  }
}

hipError_t launch_edge_rows(int64_t N, int64_t E, const int32_t* row_ptr, int32_t* rows, hipStream_t stream) {
  if (N == 0 || E == 0) return hipSuccess;
  const int64_t b = (N + 255) / 256;
  hipLaunchKernelGGL(edge_rows_kernel, dim3((unsigned)(b > 8192 ? 8192 : b)), dim3(256), 0, stream, row_ptr, (int)N,
                     (int)E, rows);
  return hipGetLastError();
}

static unsigned grid_for(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return (unsigned)(b < 1 ? 1 : (b > 8192 ? 8192 : b));
}

// steps 1-3 (the scatter also writes vec and src when their outputs are given)
static hipError_t group_by_dst(int64_t N, int64_t E, const int32_t* dst, const float* vec, const int32_t* src,
                               int32_t* row_ptr, int32_t* perm, float* vec_out, int32_t* src_out, hipStream_t stream) {
  hipLaunchKernelGGL(zero_i32_kernel, dim3(grid_for(N)), dim3(256), 0, stream, row_ptr, (int)N);
  if (E > 0)
    hipLaunchKernelGGL(dst_histogram_kernel, dim3(grid_for(E)), dim3(256), 0, stream, dst, (int)E, (int)N, row_ptr);
  hipLaunchKernelGGL(inclusive_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, row_ptr, (int)N, (int)E);
  if (E > 0)
    hipLaunchKernelGGL(scatter_by_dst_kernel, dim3(grid_for(E)), dim3(256), 0, stream, dst, vec, src, (int)E, (int)N,
                       row_ptr, perm, vec_out, src_out);
  return hipGetLastError();
}

hipError_t launch_sort_edges(int64_t N, int64_t E, const int32_t* dst, const float* vec, const int32_t* src,
                             int32_t* row_ptr, int32_t* perm, float* vec_out, int32_t* src_out, hipStream_t stream) {
  return group_by_dst(N, E, dst, vec, src, row_ptr, perm, vec_out, src_out, stream);
}

// ---------------------------------------------------------------------------
// Stable grouping by destination (LSD radix sort), for eqtp_conv_fused_ws
// ---------------------------------------------------------------------------
constexpr int kRadixMaxBits = 9;
constexpr int kRadixMaxBins = 1 << kRadixMaxBits;
constexpr int kRadixThreads = 256;
constexpr int kRadixMaxRounds = 16;
constexpr int kRadixWaves = kRadixThreads / 64;

// rounds of 256 items per workgroup: up to 16, fewer for small E so that there are about 512 tiles
static int radix_rounds(int64_t E) {
  const int64_t r = E / ((int64_t)kRadixThreads * 512);
  return r < 1 ? 1 : (r > kRadixMaxRounds ? kRadixMaxRounds : (int)r);
}

struct RadixPlan {
  int passes, bits;
};
static RadixPlan radix_plan(int64_t N) {
  int len = 0;  // bits of the largest key, N - 1
  while (len < 31 && ((int64_t)1 << len) < N) ++len;
  RadixPlan p;
  p.passes = len <= kRadixMaxBits ? 1 : (len + kRadixMaxBits - 1) / kRadixMaxBits;
  p.bits = len == 0 ? 1 : (len + p.passes - 1) / p.passes;
  return p;
}

int64_t radix_tiles(int64_t E) {
  const int64_t tile = (int64_t)kRadixThreads * radix_rounds(E);
  return (E + tile - 1) / tile;
}
// the counts [bins][tiles], the digit totals [bins] and their grand total
int64_t radix_hist_entries(int64_t E) { return (int64_t)kRadixMaxBins * (radix_tiles(E) + 1) + 1; }

// Exclusive scan of each of `rows` rows of `len` ints (row b at a + b * len) in place, one workgroup per
// row; the row's total goes to totals[b].  Chunks of 4 x 256 entries: per-thread sums, a shuffle scan in
// each wave, the wave totals through LDS, a carry between chunks.
__global__ __launch_bounds__(256) void row_exclusive_scan_kernel(int* __restrict__ a, int len,
                                                                 int* __restrict__ totals) {
  __shared__ int wsum[4];
  int* row = a + (size_t)blockIdx.x * len;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  int carry = 0;
  for (int c0 = 0; c0 < len; c0 += 1024) {
    int v[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = c0 + 4 * t + q;
      v[q] = i < len ? row[i] : 0;
      sum += v[q];
    }
    int incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int u = __shfl_up(incl, off, 64);
      if (lane >= off) incl += u;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int before = carry, all = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      before += w < wv ? wsum[w] : 0;
      all += wsum[w];
    }
    int run = before + incl - sum;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = c0 + 4 * t + q;
      if (i < len) row[i] = run;
      run += v[q];
    }
    carry += all;
    __syncthreads();  // wsum is rewritten by the next chunk
  }
  if (t == 0) totals[blockIdx.x] = carry;
}

__global__ __launch_bounds__(kRadixThreads) void radix_upsweep_kernel(const int* __restrict__ keys, int E, int N,
                                                                      int shift, int bins, int ntiles, int rounds,
                                                                      int* __restrict__ hist) {
  __shared__ int cnt[kRadixMaxBins];
  for (int b = threadIdx.x; b < bins; b += kRadixThreads) cnt[b] = 0;
  __syncthreads();
  const int base = blockIdx.x * kRadixThreads * rounds;
  for (int r = 0; r < rounds; ++r) {
    const int i = base + r * kRadixThreads + threadIdx.x;
    if (i < E) atomicAdd(&cnt[(clamp_index(keys[i], N) >> shift) & (bins - 1)], 1);
  }
  __syncthreads();
  for (int b = threadIdx.x; b < bins; b += kRadixThreads) hist[b * ntiles + blockIdx.x] = cnt[b];
}

// hist[digit][tile]: exclusive offsets within each digit; base[digit]: exclusive offsets of the digits;
// vals_in == nullptr: the values are the indices
__global__ __launch_bounds__(kRadixThreads) void radix_downsweep_kernel(const int* __restrict__ keys_in,
                                                                        const int* __restrict__ vals_in, int E,
                                                                        int N, int shift, int bits, int ntiles,
                                                                        int rounds, const int* __restrict__ hist,
                                                                        const int* __restrict__ base,
                                                                        int* __restrict__ keys_out,
                                                                        int* __restrict__ vals_out) {
  __shared__ int toff[kRadixMaxBins];             // next free place of each digit in this tile's output
  __shared__ int wcnt[kRadixWaves][kRadixMaxBins];  // this round's count of each digit per wave
  const int bins = 1 << bits;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  for (int b = t; b < bins; b += kRadixThreads) {
    toff[b] = base[b] + hist[b * ntiles + blockIdx.x];
    for (int w = 0; w < kRadixWaves; ++w) wcnt[w][b] = 0;
  }
  __syncthreads();
  const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  const int first = blockIdx.x * kRadixThreads * rounds;
  for (int r = 0; r < rounds; ++r) {
    const int i = first + r * kRadixThreads + t;
    const bool valid = i < E;
    int k = 0, v = 0, d = 0;
    if (valid) {
      k = clamp_index(keys_in[i], N);
      v = vals_in != nullptr ? vals_in[i] : i;
      d = (k >> shift) & (bins - 1);
    }
    // lanes of this wave holding an item with the same digit
    uint64_t same = __ballot(valid);
    for (int b = 0; b < bits; ++b) {
      const bool bit = (d >> b) & 1;
      const uint64_t on = __ballot(bit);
      same &= bit ? on : ~on;
    }
    const int rank = __popcll(same & below);
    if (valid && rank == 0) wcnt[wv][d] = __popcll(same);  // the group's first lane publishes its size
    __syncthreads();
    if (valid) {
      int pos = toff[d] + rank;
      for (int w = 0; w < wv; ++w) pos += wcnt[w][d];
      keys_out[pos] = k;
      vals_out[pos] = v;
    }
    __syncthreads();
    for (int b = t; b < bins; b += kRadixThreads) {
      int sum = 0;
      for (int w = 0; w < kRadixWaves; ++w) {
        sum += wcnt[w][b];
        wcnt[w][b] = 0;
      }
      toff[b] += sum;
    }
    __syncthreads();
  }
}

// row_ptr from keys sorted ascending in [0, N): every entry is written exactly once
__global__ __launch_bounds__(256) void rows_from_sorted_kernel(const int* __restrict__ keys, int E, int N,
                                                               int* __restrict__ row_ptr) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i <= E; i += gridDim.x * blockDim.x) {
    const int kp = i > 0 ? keys[i - 1] : -1;
    const int kc = i < E ? keys[i] : N;
    for (int d = kp + 1; d <= kc; ++d) row_ptr[d] = i;
  }
}

__global__ __launch_bounds__(256) void gather_sorted_kernel(const int* __restrict__ vals, int E,
                                                            const float* __restrict__ vec,
                                                            const int* __restrict__ src, float* __restrict__ vec_out,
                                                            int* __restrict__ src_out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;  // one edge per thread (the grid covers E)
  if (i >= E) return;
  const int e = clamp_index(vals[i], E);
  if (vec_out != nullptr) {
    const float a = vec[3 * (size_t)e], b = vec[3 * (size_t)e + 1], c = vec[3 * (size_t)e + 2];
    vec_out[3 * (size_t)i] = a;
    vec_out[3 * (size_t)i + 1] = b;
    vec_out[3 * (size_t)i + 2] = c;
  }
  if (src_out != nullptr) src_out[i] = src[e];
}

hipError_t launch_sort_edges_stable(int64_t N, int64_t E, const int32_t* dst, const float* vec, const int32_t* src,
                                    int32_t* row_ptr, int32_t* keys_a, int32_t* vals_a, int32_t* keys_b,
                                    int32_t* vals_b, int32_t* hist, float* vec_out, int32_t* src_out,
                                    hipStream_t stream) {
  if (E == 0) {
    hipLaunchKernelGGL(rows_from_sorted_kernel, dim3(1), dim3(256), 0, stream, keys_a, 0, (int)N, row_ptr);
    return hipGetLastError();
  }
  const RadixPlan plan = radix_plan(N);
  const int ntiles = (int)radix_tiles(E);
  const int rounds = radix_rounds(E);
  const int bins = 1 << plan.bits;
  int32_t* totals = hist + (size_t)kRadixMaxBins * ntiles;
  // the last pass writes (keys_a, vals_a)
  const int32_t* kin = dst;
  const int32_t* vin = nullptr;
  for (int p = 0; p < plan.passes; ++p) {
    const bool to_a = ((plan.passes - 1 - p) & 1) == 0;
    int32_t* kout = to_a ? keys_a : keys_b;
    int32_t* vout = to_a ? vals_a : vals_b;
    const int shift = p * plan.bits;
    hipLaunchKernelGGL(radix_upsweep_kernel, dim3(ntiles), dim3(kRadixThreads), 0, stream, kin, (int)E, (int)N,
                       shift, bins, ntiles, rounds, hist);
    hipLaunchKernelGGL(row_exclusive_scan_kernel, dim3(bins), dim3(256), 0, stream, hist, ntiles, totals);
    hipLaunchKernelGGL(row_exclusive_scan_kernel, dim3(1), dim3(256), 0, stream, totals, bins,
                       totals + kRadixMaxBins);  // the grand total goes past the totals
    hipLaunchKernelGGL(radix_downsweep_kernel, dim3(ntiles), dim3(kRadixThreads), 0, stream, kin, vin, (int)E,
                       (int)N, shift, plan.bits, ntiles, rounds, hist, totals, kout, vout);
    kin = kout;
    vin = vout;
  }
  hipLaunchKernelGGL(rows_from_sorted_kernel, dim3(grid_for(E + 1)), dim3(256), 0, stream, keys_a, (int)E, (int)N,
                     row_ptr);
  if (vec_out != nullptr || src_out != nullptr)
    hipLaunchKernelGGL(gather_sorted_kernel, dim3((unsigned)((E + 255) / 256)), dim3(256), 0, stream, vals_a,
                       (int)E, vec, src, vec_out, src_out);
  return hipGetLastError();
}

}  // namespace eqtp
