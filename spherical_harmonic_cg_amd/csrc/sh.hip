// sh.hip -- standalone real spherical harmonics of edge vectors (Batmobile
// page, section "2. register intermediate computation"), plus the zero-fill
// kernel used before atomic accumulation.
//
// One thread per edge.  Bytes per edge: 12 in, 4 (lmax+1)^2 out, so the kernel
// is bound by HBM bandwidth.  A workgroup of 256 edges stages its input
// vectors and its output rows through LDS so that every global access of a
// wavefront is one contiguous run.
#include "eqtp_device.hpp"
#include "eqtp_kernels.hpp"
#include "generated/so2_tables.inc"

namespace eqtp {

constexpr int kShBlock = 256;

// Real harmonics of degree l <= L (any L <= 6) by the Legendre-derivative
// recurrence, same convention as sh_eval (page order, Condon-Shortley phase):
//   Y_l0 = A_l0 Q_l^0(z),  Y_lm,c / Y_lm,s = A_lm Q_l^m(z) Re / Im (x + i y)^m
// for the unit vector (x, y, z), with Q_l^m = d^m P_l / dz^m:
//   Q_m^m = (2m-1)!!,  Q_{m+1}^m = (2m+1) z Q_m^m,
//   Q_l^m = ((2l-1) z Q_{l-1}^m - (l+m-1) Q_{l-2}^m) / (l-m),
// and A_lm the prefactors of gen_so2_table.py.  A zero vector gives
// (Y00, 0, ..., 0).
template <int L>
__device__ __forceinline__ void sh_eval_rec(float vx, float vy, float vz, float (&Y)[num_comp(L)]) {
  const float r2 = vx * vx + vy * vy + vz * vz;
  const bool nz = r2 > 0.0f;
  const float inv = nz ? rsqrtf(r2) : 0.0f;
  const float x = vx * inv, y = vy * inv, z = vz * inv;
  float cr[L + 1], ci[L + 1];  // (x + i y)^m
  cr[0] = 1.0f;
  ci[0] = 0.0f;
#pragma unroll
  for (int m = 1; m <= L; ++m) {
    cr[m] = fmaf(cr[m - 1], x, -ci[m - 1] * y);
    ci[m] = fmaf(ci[m - 1], x, cr[m - 1] * y);
  }
  float dfact = 1.0f;  // (2m-1)!!
#pragma unroll
  for (int m = 0; m <= L; ++m) {
    if (m > 0) dfact *= (float)(2 * m - 1);
    float q2 = 0.0f, q1 = dfact;  // Q_{l-2}^m, Q_{l-1}^m
#pragma unroll
    for (int l = m; l <= L; ++l) {
      float q;
      if (l == m) {
        q = dfact;
      } else if (l == m + 1) {
        q = (float)(2 * m + 1) * z * dfact;
      } else {
        q = ((float)(2 * l - 1) * z * q1 - (float)(l + m - 1) * q2) * (1.0f / (float)(l - m));
      }
      if (l > m) {
        q2 = q1;
        q1 = q;
      }
      const float a = eqtp_gen::kShPrefactor[l][m] * q;
      if (m == 0) {
        Y[l * l] = (l == 0 || nz) ? a : 0.0f;
      } else {
        Y[l * l + 2 * m - 1] = a * cr[m];
        Y[l * l + 2 * m] = a * ci[m];
      }
    }
  }
}

// degrees 4..6: the recurrence above, otherwise as sh_kernel
template <int L>
__global__ __launch_bounds__(kShBlock) void sh_rec_kernel(const float* __restrict__ vec, int E, float* __restrict__ Y) {
  constexpr int K = num_comp(L);
  constexpr int KP = (K % 2) ? K : K + 1;  // odd LDS row stride
  __shared__ float vin[3 * kShBlock];
  __shared__ float tile[kShBlock * KP];
  const int e0 = blockIdx.x * kShBlock;
  const int nb = min(kShBlock, E - e0);
  for (int i = threadIdx.x; i < 3 * nb; i += kShBlock) vin[i] = vec[(size_t)3 * e0 + i];
  __syncthreads();
  const int t = threadIdx.x;
  if (t < nb) {
    float Yv[K];
    sh_eval_rec<L>(vin[3 * t], vin[3 * t + 1], vin[3 * t + 2], Yv);
#pragma unroll
    for (int k = 0; k < K; ++k) tile[t * KP + k] = Yv[k];
  }
  __syncthreads();
  float* yb = Y + (size_t)e0 * K;
  for (int i = t; i < nb * K; i += kShBlock) yb[i] = tile[(i / K) * KP + (i % K)];
}

template <int L>
__global__ __launch_bounds__(kShBlock) void sh_kernel(const float* __restrict__ vec, int E, float* __restrict__ Y) {
  constexpr int K = num_comp(L);
  constexpr int KP = (K % 2) ? K : K + 1;  // odd LDS row stride
  __shared__ float vin[3 * kShBlock];
  __shared__ float tile[kShBlock * KP];
  const int e0 = blockIdx.x * kShBlock;
  const int nb = min(kShBlock, E - e0);
  for (int i = threadIdx.x; i < 3 * nb; i += kShBlock) vin[i] = vec[(size_t)3 * e0 + i];
  __syncthreads();
  const int t = threadIdx.x;
  float Yv[16];
  if (t < nb) {
    sh_eval<L>(vin[3 * t], vin[3 * t + 1], vin[3 * t + 2], Yv);
#pragma unroll
    for (int k = 0; k < K; ++k) tile[t * KP + k] = Yv[k];
  }
  __syncthreads();
  float* yb = Y + (size_t)e0 * K;
  for (int i = t; i < nb * K; i += kShBlock) yb[i] = tile[(i / K) * KP + (i % K)];
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, long long n) {
  const long long n4 = n / 4;
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
    reinterpret_cast<f4*>(p)[i] = f4{0.f, 0.f, 0.f, 0.f};
  for (long long i = n4 * 4 + (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0.0f;
}

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  long long blocks = (n / 4 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, (long long)n);
  return hipGetLastError();
}

hipError_t launch_sh(const float* vec, int64_t E, int lmax, float* Y, hipStream_t stream) {
  if (E == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((E + kShBlock - 1) / kShBlock);
  switch (lmax) {
    case 0: hipLaunchKernelGGL(sh_kernel<0>, dim3(blocks), dim3(kShBlock), 0, stream, vec, (int)E, Y); break;
    case 1: hipLaunchKernelGGL(sh_kernel<1>, dim3(blocks), dim3(kShBlock), 0, stream, vec, (int)E, Y); break;
    case 2: hipLaunchKernelGGL(sh_kernel<2>, dim3(blocks), dim3(kShBlock), 0, stream, vec, (int)E, Y); break;
    case 3: hipLaunchKernelGGL(sh_kernel<3>, dim3(blocks), dim3(kShBlock), 0, stream, vec, (int)E, Y); break;
    case 4: hipLaunchKernelGGL(sh_rec_kernel<4>, dim3(blocks), dim3(kShBlock), 0, stream, vec, (int)E, Y); break;
    case 5: hipLaunchKernelGGL(sh_rec_kernel<5>, dim3(blocks), dim3(kShBlock), 0, stream, vec, (int)E, Y); break;
    case 6: hipLaunchKernelGGL(sh_rec_kernel<6>, dim3(blocks), dim3(kShBlock), 0, stream, vec, (int)E, Y); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace eqtp
