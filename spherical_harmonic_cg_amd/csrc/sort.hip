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
// The convolution over edges in any order (eqtp_conv_fused_ws) stages step 3's
// indices in its workspace and adds
//   4. one wavefront per row puts the row's indices in increasing order (each
//      index's rank among the row's indices is its place) and gathers vec and
//      src in that order: the edges of a row keep their input order, so the
//      grouping, and the convolution after it, do not depend on the atomics.
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

// Step 4: one wavefront per row (persistent waves, rows strided).  Lane i of
// chunk k holds the row's index at slot 64k + i; its rank is the number of
// the row's indices below it, counted against each chunk held in a register
// and broadcast lane by lane.  Indices are distinct (one per edge).  The
// outputs must not alias `staged`.
constexpr int kRowWaves = 4;
__global__ __launch_bounds__(kRowWaves * 64) void row_order_kernel(const int* __restrict__ row_ptr, int N, int E,
                                                                   const int* __restrict__ staged,
                                                                   const float* __restrict__ vec,
                                                                   const int* __restrict__ src,
                                                                   float* __restrict__ vec_out,
                                                                   int* __restrict__ src_out) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * kRowWaves + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * kRowWaves;
  for (int r = wave; r < N; r += nwaves) {
    const int b = min(max(row_ptr[r], 0), E);
    const int e = min(max(row_ptr[r + 1], b), E);
    const int len = e - b;
    for (int c0 = 0; c0 < len; c0 += 64) {
      const bool mine_ok = c0 + lane < len;
      const int mine = mine_ok ? staged[b + c0 + lane] : 0;
      int rank = 0;
      for (int k0 = 0; k0 < len; k0 += 64) {
        const int other = k0 + lane < len ? staged[b + k0 + lane] : 0x7fffffff;
        const int n = min(64, len - k0);
        for (int j = 0; j < n; ++j) rank += __builtin_amdgcn_readlane(other, j) < mine ? 1 : 0;
      }
      if (mine_ok) {
        const int slot = b + rank;
        const int ei = clamp_index(mine, E);
        vec_out[3 * (size_t)slot] = vec[3 * (size_t)ei];
        vec_out[3 * (size_t)slot + 1] = vec[3 * (size_t)ei + 1];
        vec_out[3 * (size_t)slot + 2] = vec[3 * (size_t)ei + 2];
        src_out[slot] = src[ei];
      }
    }
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

hipError_t launch_sort_edges_ordered(int64_t N, int64_t E, const int32_t* dst, const float* vec, const int32_t* src,
                                     int32_t* row_ptr, int32_t* staged, float* vec_out, int32_t* src_out,
                                     hipStream_t stream) {
  hipError_t err = group_by_dst(N, E, dst, nullptr, nullptr, row_ptr, staged, nullptr, nullptr, stream);
  if (err != hipSuccess || E == 0) return err;
  const int64_t rb = (N + kRowWaves - 1) / kRowWaves;
  const unsigned rgrid = (unsigned)(rb < 1 ? 1 : (rb > 4096 ? 4096 : rb));
  hipLaunchKernelGGL(row_order_kernel, dim3(rgrid), dim3(kRowWaves * 64), 0, stream, row_ptr, (int)N, (int)E,
                     staged, vec, src, vec_out, src_out);
  return hipGetLastError();
}

}  // namespace eqtp
