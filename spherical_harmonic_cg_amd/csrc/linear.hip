// linear.hip -- per-l channel linear out[n,c',l m] = sum_c W[l,c',c] h[n,c,l m]
// on the matrix cores (the one dense contraction of the path).
//
// A workgroup (4 waves) takes 16 consecutive nodes -- one contiguous
// 16*C*K-float block of h -- loads it coalesced and stores it in LDS
// transposed to [m][node][c].  Work items are (component m, 16-row tile of
// output channels); for each, the 16x16 output tile D[c'][node] is
//   fp32 mode: sum over 16-channel blocks of 4 v_mfma_f32_16x16x4_f32, lane
//              (i = l%16, k = l/16) supplying W[c'0+i][ci0+4k+s] and
//              h[node i][ci0+4k+s][m] for s = 0..3 (one 16-byte read each);
//   bf16 mode: sum over 32-channel blocks of v_mfma_f32_16x16x32_bf16 with
//              8 consecutive input channels per lane, both operands rounded
//              to bfloat16 (nearest even) as they are loaded.
// Results wait in registers until every wave is done with the input tile,
// then go through LDS (reusing it) to a coalesced store.  Bytes per node:
// 8 C K (read h, write out); flops 2 C^2 K: bound by HBM bandwidth.
#include "eqtp_device.hpp"
#include "eqtp_kernels.hpp"

namespace eqtp {

template <int L, int C, bool BF16>
struct LinCfg {
  static constexpr int K = num_comp(L);
  static constexpr int TN = 16;                  // nodes per workgroup
  static constexpr int CS = C + 4;               // LDS row stride (floats), 16-byte aligned
  static constexpr int CT = (C + 15) / 16;       // output channel tiles
  static constexpr int ITEMS = K * CT;
  static constexpr int WAVES = 4;
  static constexpr int IPW = (ITEMS + WAVES - 1) / WAVES;
  static constexpr int LDS_IN = K * TN * CS;
  static constexpr int LDS_OUT = TN * C * K;
  static constexpr int LDS = LDS_IN > LDS_OUT ? LDS_IN : LDS_OUT;
  static_assert(LDS * 4 <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ int l_of(int m) { return m >= 9 ? 3 : (m >= 4 ? 2 : (m >= 1 ? 1 : 0)); }

template <int L, int C, bool BF16>
__global__ __launch_bounds__(256) void linear_kernel(int N, const float* __restrict__ h, const float* __restrict__ W,
                                                     float* __restrict__ out) {
  using Cfg = LinCfg<L, C, BF16>;
  constexpr int K = Cfg::K;
  constexpr int TN = Cfg::TN;
  constexpr int CS = Cfg::CS;
  __shared__ __attribute__((aligned(16))) float lds[Cfg::LDS];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int n0 = blockIdx.x * TN;
  const int nv = min(TN, N - n0);
  const size_t base = (size_t)n0 * C * K;

  // 1. tile load, transposed into lds[m][node][c]
  for (int f = threadIdx.x; f < TN * C * K; f += 256) {
    const int n = f / (C * K);
    const int rem = f - n * (C * K);
    const int c = rem / K;
    const int m = rem - c * K;
    lds[(m * TN + n) * CS + c] = n < nv ? h[base + f] : 0.0f;
  }
  __syncthreads();

  // 2. matrix-core products; results held in registers
  const int i16 = lane & 15;
  const int kq = lane >> 4;
  f4 res[Cfg::IPW];
#pragma unroll
  for (int q = 0; q < Cfg::IPW; ++q) {
    res[q] = f4{0.f, 0.f, 0.f, 0.f};
    const int item = wv + q * Cfg::WAVES;
    if (item < Cfg::ITEMS) {
      const int m = item / Cfg::CT;
      const int ct = item - m * Cfg::CT;
      const int l = l_of(m);
      const int co = ct * 16 + i16;  // output channel supplied by this lane (A rows)
      const bool co_ok = co < C;
      const float* wrow = W + ((size_t)l * C + (co_ok ? co : 0)) * C;
      const float* hrow = lds + (m * TN + i16) * CS;
      f4 acc = f4{0.f, 0.f, 0.f, 0.f};
      if constexpr (!BF16) {
#pragma unroll
        for (int ci0 = 0; ci0 < C; ci0 += 16) {
          const int cb = ci0 + 4 * kq;
          f4 a4 = f4{0.f, 0.f, 0.f, 0.f}, b4 = f4{0.f, 0.f, 0.f, 0.f};
          if (cb < C) {
            if (co_ok) a4 = *reinterpret_cast<const f4*>(wrow + cb);
            b4 = *reinterpret_cast<const f4*>(hrow + cb);
          }
#pragma unroll
          for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[s], b4[s], acc, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int ci0 = 0; ci0 < C; ci0 += 32) {
          const int cb = ci0 + 8 * kq;
          bf16x8 a8, b8;
          f4 a0 = f4{0.f, 0.f, 0.f, 0.f}, a1 = a0, b0 = a0, b1 = a0;
          if (cb < C) {
            if (co_ok) {
              a0 = *reinterpret_cast<const f4*>(wrow + cb);
              a1 = *reinterpret_cast<const f4*>(wrow + cb + 4);
            }
            b0 = *reinterpret_cast<const f4*>(hrow + cb);
            b1 = *reinterpret_cast<const f4*>(hrow + cb + 4);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            a8[j] = to_bf16(a0[j]);
            a8[4 + j] = to_bf16(a1[j]);
            b8[j] = to_bf16(b0[j]);
            b8[4 + j] = to_bf16(b1[j]);
          }
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, b8, acc, 0, 0, 0);
        }
      }
      res[q] = acc;
    }
  }
  __syncthreads();

  // 3. D[c' = ct*16 + 4 kq + v][node = i16] -> lds[node][c'][m] (global layout)
#pragma unroll
  for (int q = 0; q < Cfg::IPW; ++q) {
    const int item = wv + q * Cfg::WAVES;
    if (item < Cfg::ITEMS) {
      const int m = item / Cfg::CT;
      const int ct = item - m * Cfg::CT;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int co = ct * 16 + 4 * kq + v;
        if (co < C) lds[(i16 * C + co) * K + m] = res[q][v];
      }
    }
  }
  __syncthreads();

  // 4. coalesced store of the valid nodes
  const int nf4 = nv * C * K / 4;
  f4* ob = reinterpret_cast<f4*>(out + base);
  const f4* tb = reinterpret_cast<const f4*>(lds);
  for (int i = threadIdx.x; i < nf4; i += 256) ob[i] = tb[i];
}

template <int L, int C, bool BF16>
static hipError_t launch_linear_t(int64_t N, const float* h, const float* W, float* out, hipStream_t stream) {
  const unsigned blocks = (unsigned)((N + 15) / 16);
  hipLaunchKernelGGL((linear_kernel<L, C, BF16>), dim3(blocks), dim3(256), 0, stream, (int)N, h, W, out);
  return hipGetLastError();
}

template <int L, bool BF16>
static hipError_t dispatch_linear_c(int64_t N, int C, const float* h, const float* W, float* out, hipStream_t s) {
  switch (C) {
    case 8: return launch_linear_t<L, 8, BF16>(N, h, W, out, s);
    case 16: return launch_linear_t<L, 16, BF16>(N, h, W, out, s);
    case 32: return launch_linear_t<L, 32, BF16>(N, h, W, out, s);
    case 64: return launch_linear_t<L, 64, BF16>(N, h, W, out, s);
    case 128: return launch_linear_t<L, 128, BF16>(N, h, W, out, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_linear(int64_t N, int C, int lmax, int bf16, const float* h, const float* W, float* out,
                         hipStream_t stream) {
  if (N == 0) return hipSuccess;
  switch (lmax * 2 + (bf16 ? 1 : 0)) {
    case 0: return dispatch_linear_c<0, false>(N, C, h, W, out, stream);
    case 1: return dispatch_linear_c<0, true>(N, C, h, W, out, stream);
    case 2: return dispatch_linear_c<1, false>(N, C, h, W, out, stream);
    case 3: return dispatch_linear_c<1, true>(N, C, h, W, out, stream);
    case 4: return dispatch_linear_c<2, false>(N, C, h, W, out, stream);
    case 5: return dispatch_linear_c<2, true>(N, C, h, W, out, stream);
    case 6: return dispatch_linear_c<3, false>(N, C, h, W, out, stream);
    case 7: return dispatch_linear_c<3, true>(N, C, h, W, out, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace eqtp
