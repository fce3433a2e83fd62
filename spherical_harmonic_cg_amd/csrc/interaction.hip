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
// Both layers are products with the edges as rows, so a wave takes 16 edges
// at a time and runs them on v_mfma_f32_16x16x4_f32 (fp32 products and
// sums): layer 1 is [16 x 8] x [8 x 64] (8 products), layer 2 [16 x 64] x
// [64 x 64] (64 products), with W1 and W2 held in registers as B operands
// for the whole kernel.  Lane (i, g) of the A operand supplies edge i and
// inputs g, g + 4, ...; the radial functions of edge i are evaluated by the
// four lanes that feed its row.  Between the layers, and before the store,
// the results go through a 16 x 64 LDS tile in the order unit 4 s + q at
// q * 16 + s, which is both the layout the second layer's A operand reads
// contiguously and the phi layout above, so every global store is a
// coalesced 16-byte one.  About 4.6k multiply-adds per edge against the path
// weights' 94k at P = 23, C = 64.
#include "eqtp_device.hpp"
#include "eqtp_kernels.hpp"

namespace eqtp {

constexpr int kMlpHidden = 64;
constexpr int kMlpBasis = 8;
constexpr int kMlpWaves = 4;
constexpr int kMlpRow = kMlpHidden + 4;  // LDS row stride (floats): rows start 4 banks apart

__device__ __forceinline__ float silu(float t) { return t / (1.0f + __expf(-t)); }

// position of hidden unit h = 4 s + q in an LDS row and in phi: q * 16 + s
__device__ __forceinline__ int mlp_slot(int h) { return (h & 3) * 16 + (h >> 2); }

__global__ __launch_bounds__(kMlpWaves * kWave) void radial_mlp_kernel(int E, const float* __restrict__ vec,
                                                                       const float* __restrict__ W1,
                                                                       const float* __restrict__ W2,
                                                                       float* __restrict__ phi, float inv_rc,
                                                                       float scale) {
  __shared__ __attribute__((aligned(16))) float tile[kMlpWaves][16 * kMlpRow];
  const int lane = threadIdx.x & 63;
  const int i16 = lane & 15;  // A row (edge) / B and D column
  const int kq = lane >> 4;   // A / B k group; D rows 4 kq .. 4 kq + 3
  float* const t = tile[threadIdx.x >> 6];
  // B operands: w1b[s][j] = W1[4 s + kq, 16 j + i16], w2b[s][j] = W2[4 s + kq, 16 j + i16]
  float w1b[2][4], w2b[16][4];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int j = 0; j < 4; ++j) w1b[s][j] = W1[(4 * s + kq) * kMlpHidden + 16 * j + i16];
#pragma unroll
  for (int s = 0; s < 16; ++s)
#pragma unroll
    for (int j = 0; j < 4; ++j) w2b[s][j] = W2[(4 * s + kq) * kMlpHidden + 16 * j + i16];
  const int nbatch = (E + 15) / 16;
  const int nwaves = gridDim.x * kMlpWaves;
  for (int b = blockIdx.x * kMlpWaves + (threadIdx.x >> 6); b < nbatch; b += nwaves) {
    const int e = 16 * b + i16;
    float R[kMlpBasis];
#pragma unroll
    for (int k = 0; k < kMlpBasis; ++k) R[k] = 0.0f;
    if (e < E) {
      const float vx = vec[3 * (size_t)e], vy = vec[3 * (size_t)e + 1], vz = vec[3 * (size_t)e + 2];
      radial_basis<kMlpBasis>(sqrtf(vx * vx + vy * vy + vz * vz), inv_rc, R);
    }
    const float r0 = kq == 0 ? R[0] : (kq == 1 ? R[1] : (kq == 2 ? R[2] : R[3]));
    const float r1 = kq == 0 ? R[4] : (kq == 1 ? R[5] : (kq == 2 ? R[6] : R[7]));
    // layer 1: a[edge 4 kq + v][unit 16 j + i16] = SiLU(acc[j][v]) -> LDS
    f4 acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(r0, w1b[0][j], f4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(r1, w1b[1][j], acc[j], 0, 0, 0);
    }
    wave_lds_sync();  // the previous batch's tile has been read
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) t[(4 * kq + v) * kMlpRow + mlp_slot(16 * j + i16)] = silu(acc[j][v]);
    wave_lds_sync();
    // layer 2: A operand of lane (edge i16, kq) = units kq, 4 + kq, ..., 60 + kq: 16 contiguous floats
    f4 av[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) av[q] = *reinterpret_cast<const f4*>(t + i16 * kMlpRow + kq * 16 + 4 * q);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 16; ++s)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s >> 2][s & 3], w2b[s][j], acc[j], 0, 0, 0);
    wave_lds_sync();  // every lane has read its A operands
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) t[(4 * kq + v) * kMlpRow + mlp_slot(16 * j + i16)] = silu(acc[j][v]) * scale;
    wave_lds_sync();
    // 16 rows of 64 floats leave as 256 coalesced 16-byte stores (four per lane)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int f = 64 * q + lane;  // 16-byte piece f: row f / 16, columns 4 (f % 16) .. 4 (f % 16) + 3
      const int r = f >> 4, c4 = f & 15;
      if (16 * b + r < E)
        *reinterpret_cast<f4*>(phi + (size_t)(16 * b + r) * kMlpHidden + 4 * c4) =
            *reinterpret_cast<const f4*>(t + r * kMlpRow + 4 * c4);
    }
  }
}

hipError_t launch_radial_mlp(int64_t E, const float* vec, float r_cut, const float* W1, const float* W2, float* phi,
                             float scale, hipStream_t stream) {
  if (E == 0) return hipSuccess;
  const int64_t nbatch = (E + 15) / 16;
  const int64_t want = 8LL * num_cus();  // workgroups of four waves, eight per CU at most
  const int64_t need = (nbatch + kMlpWaves - 1) / kMlpWaves;
  const int64_t blocks = need < want ? need : want;
  hipLaunchKernelGGL(radial_mlp_kernel, dim3((unsigned)blocks), dim3(kMlpWaves * kWave), 0, stream, (int)E, vec, W1,
                     W2, phi, 1.0f / r_cut, scale);
  return hipGetLastError();
}

}  // namespace eqtp
