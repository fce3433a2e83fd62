// check.hip -- the graph checks behind eqtp_check_graph and the library's
// debug mode: every index the kernels would clamp, the CSR row pointers they
// rely on, and the edge vectors, read once on the GPU and summarised in a
// small report of integer counts (so the report does not depend on the order
// in which threads finish).
//
// Report words (kCheckWords int32):
//   0  edges whose src is outside [0, N)
//   1  edges whose dst is outside [0, N)
//   2  rows r with row_ptr[r + 1] < row_ptr[r]
//   3  endpoint faults: row_ptr[0] != 0 and row_ptr[N] != E count one each
//   4  edges e whose dst differs from the row that row_ptr puts e in
//   5  edges with a non-finite vector component
//   6  smallest edge index counted in words 0, 1, 4 or 5 (-1 if none)
//   7  smallest row index counted in word 2 (-1 if none)
#include "eqtp_device.hpp"
#include "eqtp_kernels.hpp"

namespace eqtp {

namespace {

constexpr int kCheckBlock = 256;

__global__ void check_init_kernel(int32_t* __restrict__ report) {
  const int i = threadIdx.x;
  if (i < kCheckWords) report[i] = i >= 6 ? 0x7fffffff : 0;  // no index yet (indices are below 2^31 - 1)
}

// sum over the wavefront (64 lanes) of a per-lane count
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = min(v, __shfl_xor(v, off, 64));
  return v;
}

// the row whose CSR range holds edge e: the largest r in [0, N) with
// row_ptr[r] <= e (empty rows are passed over); every read stays in [0, N)
__device__ __forceinline__ int row_of(const int32_t* __restrict__ row_ptr, int N, int e) {
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    const int mid = lo + (hi - lo + 1) / 2;
    if (row_ptr[mid] <= e) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(kCheckBlock) void check_graph_kernel(int N, int E, const int32_t* __restrict__ row_ptr,
                                                                  const int32_t* __restrict__ src,
                                                                  const int32_t* __restrict__ dst,
                                                                  const float* __restrict__ vec,
                                                                  int32_t* __restrict__ report) {
  constexpr int kNone = 0x7fffffff;
  int n_src = 0, n_dst = 0, n_dec = 0, n_end = 0, n_row = 0, n_vec = 0;
  int first_e = kNone, first_r = kNone;
  const long long total = max((long long)E, (long long)N + 1);
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long ii = (long long)blockIdx.x * blockDim.x + threadIdx.x; ii < total; ii += stride) {
    const int i = (int)ii;  // below 2^31: E and N are at most 2^31 - 1, and i == N only on the row side
    if (i < E) {
      bool bad = false;
      if (src) {
        const int s = src[i];
        if (s < 0 || s >= N) {
          ++n_src;
          bad = true;
        }
      }
      if (dst) {
        const int d = dst[i];
        if (d < 0 || d >= N) {
          ++n_dst;
          bad = true;
        }
        if (row_ptr && N > 0 && d != row_of(row_ptr, N, i)) {
          ++n_row;
          bad = true;
        }
      }
      if (vec) {
        const float a = vec[3 * (size_t)i], b = vec[3 * (size_t)i + 1], c = vec[3 * (size_t)i + 2];
        if (!(isfinite(a) && isfinite(b) && isfinite(c))) {
          ++n_vec;
          bad = true;
        }
      }
      if (bad) first_e = min(first_e, i);
    }
    if (row_ptr && i <= N) {
      if (i < N && row_ptr[i + 1] < row_ptr[i]) {
        ++n_dec;
        first_r = min(first_r, i);
      }
      if (i == 0 && row_ptr[0] != 0) ++n_end;
      if (i == N && row_ptr[N] != E) ++n_end;
    }
  }
  n_src = wave_sum(n_src);
  n_dst = wave_sum(n_dst);
  n_dec = wave_sum(n_dec);
  n_end = wave_sum(n_end);
  n_row = wave_sum(n_row);
  n_vec = wave_sum(n_vec);
  first_e = wave_min(first_e);
  first_r = wave_min(first_r);
  if ((threadIdx.x & 63) == 0) {
    if (n_src) atomicAdd(report + 0, n_src);
    if (n_dst) atomicAdd(report + 1, n_dst);
    if (n_dec) atomicAdd(report + 2, n_dec);
    if (n_end) atomicAdd(report + 3, n_end);
    if (n_row) atomicAdd(report + 4, n_row);
    if (n_vec) atomicAdd(report + 5, n_vec);
    if (first_e != kNone) atomicMin(report + 6, first_e);
    if (first_r != kNone) atomicMin(report + 7, first_r);
  }
}

// words 6 and 7 hold 2^31 - 1 where no index was counted; report -1 there
__global__ void check_finish_kernel(int32_t* __restrict__ report) {
  const int i = threadIdx.x;
  if ((i == 6 || i == 7) && report[i] == 0x7fffffff) report[i] = -1;
}

}  // namespace

hipError_t launch_check_graph(int64_t N, int64_t E, const int32_t* row_ptr, const int32_t* src, const int32_t* dst,
                              const float* vec, int32_t* report, hipStream_t stream) {
  hipLaunchKernelGGL(check_init_kernel, dim3(1), dim3(64), 0, stream, report);
  const int64_t total = E > N + 1 ? E : N + 1;
  const int64_t blocks = (total + kCheckBlock - 1) / kCheckBlock;
  const int grid = (int)(blocks < 4096 ? blocks : 4096);
  hipLaunchKernelGGL(check_graph_kernel, dim3(grid), dim3(kCheckBlock), 0, stream, (int)N, (int)E, row_ptr, src,
                     dst, vec, report);
  hipLaunchKernelGGL(check_finish_kernel, dim3(1), dim3(64), 0, stream, report);
  return hipGetLastError();
}

}  // namespace eqtp
