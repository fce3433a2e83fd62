// interaction.hip -- the radial network of the interaction layer: for every
// edge, the 8 radial functions of its length (as for the radial weights) go
// through two hidden layers of width 64 with SiLU and no bias,
//   a[k]      = SiLU(sum_b R_b W1[b, k]),
//   phi[e, k] = SiLU(sum_j a[j] W2[j, k]) * scale,
// SiLU(t) = t / (1 + exp(-t)).  The last layer of the network (64 -> P*C) is
// not here: the edge-aligned radial kernel applies it on the matrix cores as
// it builds each edge's path weights, so the [E, P*C] weights never reach
// memory.  phi is written as [E][4][16] (unit k = 4 i + q at q * 16 + i),
// the order in which that kernel's lane groups read it.
//
// Lane k of a wave is hidden unit k; the wave walks a run of edges one at a
// time.  W1's column and W2's column of the lane's unit are held in
// registers (8 + 64 values); a[j] reaches every lane through v_readlane, so
// the second layer is 64 FMAs per lane with a wave-uniform operand.  The
// network is a small fraction of the layer's work (about 4.6k FMAs per edge
// against the path weights' 94k at P = 23, C = 64).
#include "eqtp_device.hpp"
#include "eqtp_kernels.hpp"

namespace eqtp {

constexpr int kMlpHidden = 64;
constexpr int kMlpBasis = 8;
constexpr int kMlpWaves = 4;
constexpr int kMlpRun = 32;  // edges per wave and run

__device__ __forceinline__ float silu(float t) { return t / (1.0f + __expf(-t)); }

constexpr int kMlpIlp = 4;  // edges in flight per lane (independent FMA chains)

__global__ __launch_bounds__(kMlpWaves * kWave) void radial_mlp_kernel(int E, const float* __restrict__ vec,
                                                                       const float* __restrict__ W1,
                                                                       const float* __restrict__ W2,
                                                                       float* __restrict__ phi, float inv_rc,
                                                                       float scale) {
  const int k = threadIdx.x & 63;  // hidden unit
  float w1[kMlpBasis], w2[kMlpHidden];
#pragma unroll
  for (int b = 0; b < kMlpBasis; ++b) w1[b] = W1[b * kMlpHidden + k];
#pragma unroll
  for (int jj = 0; jj < kMlpHidden; ++jj) w2[jj] = W2[jj * kMlpHidden + k];
  const int slot = (k & 3) * 16 + (k >> 2);  // where unit k = 4 i + q is stored: q * 16 + i
  const int nruns = (E + kMlpRun - 1) / kMlpRun;
  const int wave = blockIdx.x * kMlpWaves + (threadIdx.x >> 6);
  const int nwaves = gridDim.x * kMlpWaves;
  for (int run = wave; run < nruns; run += nwaves) {
    const int e_end = min(E, (run + 1) * kMlpRun);
    // kMlpIlp edges at a time; slots past the run's end repeat its last edge and are not stored
    for (int e0 = run * kMlpRun; e0 < e_end; e0 += kMlpIlp) {
      float a[kMlpIlp], t[kMlpIlp];
#pragma unroll
      for (int u = 0; u < kMlpIlp; ++u) {
        const int e = min(e0 + u, e_end - 1);
        const float vx = vec[3 * (size_t)e], vy = vec[3 * (size_t)e + 1], vz = vec[3 * (size_t)e + 2];
        float R[kMlpBasis];
        radial_basis<kMlpBasis>(sqrtf(vx * vx + vy * vy + vz * vz), inv_rc, R);
        float acc = 0.0f;
#pragma unroll
        for (int b = 0; b < kMlpBasis; ++b) acc = fmaf(R[b], w1[b], acc);
        a[u] = silu(acc);
        t[u] = 0.0f;
      }
#pragma unroll
      for (int jj = 0; jj < kMlpHidden; ++jj)
#pragma unroll
        for (int u = 0; u < kMlpIlp; ++u)
          t[u] = fmaf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, a[u]), jj)), w2[jj],
                      t[u]);
#pragma unroll
      for (int u = 0; u < kMlpIlp; ++u)
        if (e0 + u < e_end) phi[(size_t)(e0 + u) * kMlpHidden + slot] = silu(t[u]) * scale;
    }
  }
}

hipError_t launch_radial_mlp(int64_t E, const float* vec, float r_cut, const float* W1, const float* W2, float* phi,
                             float scale, hipStream_t stream) {
  if (E == 0) return hipSuccess;
  const int64_t runs = (E + kMlpRun - 1) / kMlpRun;
  const int64_t want = 8LL * num_cus();  // two workgroups of four waves per CU
  const int64_t blocks = (runs + kMlpWaves - 1) / kMlpWaves < want ? (runs + kMlpWaves - 1) / kMlpWaves : want;
  hipLaunchKernelGGL(radial_mlp_kernel, dim3((unsigned)blocks), dim3(kMlpWaves * kWave), 0, stream, (int)E, vec, W1,
                     W2, phi, 1.0f / r_cut, scale);
  return hipGetLastError();
}

}  // namespace eqtp
