// conv_edge.hip -- fused convolution evaluated edge by edge on the vector ALUs.
//
// Used for unsorted edges (messages summed into dst with fp32 atomics), for
// per-edge radial weights, and, on request, for dst-sorted fixed-weight
// edges.  Per edge (Batmobile page, sections "2. register intermediate
// computation" and "3. operator fusion"): read the edge vector and source
// index once, evaluate the harmonics in registers, then for every path p
//   K_p[mu3,mu1] = sum_mu2 C^p[mu1,mu2,mu3] Y_mu2        (channel independent)
//   t[mu3]       = sum_mu1 K_p[mu3,mu1] x[src,c,mu1]
//   acc[c,mu3]  += w_e[p,c] t[mu3]
// with the coefficients folded into the instruction stream (compile-time
// table walk).  Messages live in registers only.
//
// Lane mapping: lane = channel (C <= 64: G = 64/C edges in flight per wave,
// one per lane group; C = 128: two channels per lane).
//   * sorted: one wavefront per destination row; the row's edges are dealt
//     round-robin to the lane groups and the groups are combined at the end
//     with cross-lane xor shuffles -- no atomics, deterministic;
//   * unsorted: each wave takes a contiguous run of edges and adds every
//     message into out[dst] with global fp32 atomics (out zero-filled first).
// Radial weights: w_e[p,c] = sum_n R_n(|vec_e|) W[n, p*C + c] with the
// radial basis of eqtp_device.hpp.
// XB: the node features are bfloat16 in memory (widened exactly to fp32 on
// load); every product and sum, and the atomics, stay fp32.
// OB (unsorted edges only): out is bfloat16; each message is rounded to bf16
// (nearest even) and added with packed two-element bf16 atomics, half the
// atomic operations of the fp32 output.
#include <type_traits>

#include "eqtp_device.hpp"
#include "eqtp_kernels.hpp"

namespace eqtp {

template <int C>
struct EdgeCfg {
  static constexpr int CPL = C > 64 ? C / 64 : 1;  // channels per lane
  static constexpr int CL = C / CPL;               // lanes per edge group
  static constexpr int G = kWave / CL;             // edge groups per wave
  static constexpr int WAVES = 4;
  static constexpr int THREADS = WAVES * kWave;
  static constexpr int EPW = 16 * G;               // edges per wave, unsorted mode
};

constexpr int kRadialBasis = 8;

template <int L, int PS, int C, bool RADIAL, bool XB = false>
struct EdgeMsg {
  typedef std::conditional_t<XB, __bf16, float> XT;  // element type of x in memory
  using T = Tables<L, PS>;
  using Cfg = EdgeCfg<C>;
  static constexpr int K = num_comp(L);

  // acc[j][mu3] += message of edge e for channels cl + j*CL
  __device__ __forceinline__ static void run(int e, int N, int cl, const float* __restrict__ vec,
                                             const int* __restrict__ src, const XT* __restrict__ x,
                                             const float* __restrict__ w, const float (&wreg)[Cfg::CPL][T::P],
                                             float inv_rc, float (&acc)[Cfg::CPL][K]) {
    const float vx = vec[3 * (size_t)e], vy = vec[3 * (size_t)e + 1], vz = vec[3 * (size_t)e + 2];
    const int s = clamp_index(src[e], N);
    float Y[16];
    sh_eval<L>(vx, vy, vz, Y);
    float R[kRadialBasis];
    if constexpr (RADIAL) radial_basis<kRadialBasis>(sqrtf(vx * vx + vy * vy + vz * vz), inv_rc, R);
    float xv[Cfg::CPL][K];
#pragma unroll
    for (int j = 0; j < Cfg::CPL; ++j) {
      const XT* xp = x + ((size_t)s * C + cl + j * Cfg::CL) * K;
      if constexpr (K % 4 == 0 && !XB) {
#pragma unroll
        for (int q = 0; q < K / 4; ++q) {
          const f4 t4 = reinterpret_cast<const f4*>(xp)[q];
          xv[j][4 * q] = t4[0];
          xv[j][4 * q + 1] = t4[1];
          xv[j][4 * q + 2] = t4[2];
          xv[j][4 * q + 3] = t4[3];
        }
      } else if constexpr (K % 4 == 0) {
        // four bf16 values per 8-byte load; a bf16 value is the upper half of the fp32 with the same bits
#pragma unroll
        for (int q = 0; q < K / 4; ++q) {
          const uint2 t2 = reinterpret_cast<const uint2*>(xp)[q];
          xv[j][4 * q] = __uint_as_float(t2.x << 16);
          xv[j][4 * q + 1] = __uint_as_float(t2.x & 0xffff0000u);
          xv[j][4 * q + 2] = __uint_as_float(t2.y << 16);
          xv[j][4 * q + 3] = __uint_as_float(t2.y & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int k = 0; k < K; ++k) xv[j][k] = (float)xp[k];
      }
    }
    float kacc = 0.0f;
    float t[Cfg::CPL];
    float we[Cfg::CPL];
    static_for<0, T::NT>([&](auto ii) {
      constexpr int i = decltype(ii)::value;
      constexpr eqtp_gen::CgTerm tm = T::by_path[i];
      constexpr bool p_first = i == 0 || T::by_path[i - 1].p != tm.p;
      constexpr bool pm_first = p_first || T::by_path[i - 1].mu3 != tm.mu3;
      constexpr bool k_first = pm_first || T::by_path[i - 1].mu1 != tm.mu1;
      constexpr bool p_last = i + 1 == T::NT || T::by_path[i + 1].p != tm.p;
      constexpr bool pm_last = p_last || T::by_path[i + 1].mu3 != tm.mu3;
      constexpr bool k_last = pm_last || T::by_path[i + 1].mu1 != tm.mu1;
      if constexpr (p_first) {
#pragma unroll
        for (int j = 0; j < Cfg::CPL; ++j) {
          if constexpr (RADIAL) {
            float a = 0.0f;
#pragma unroll
            for (int b = 0; b < kRadialBasis; ++b)
              a = fmaf(R[b], w[(size_t)b * T::P * C + tm.p * C + cl + j * Cfg::CL], a);
            we[j] = a;
          } else {
            we[j] = wreg[j][tm.p];
          }
        }
      }
      if constexpr (pm_first) {
#pragma unroll
        for (int j = 0; j < Cfg::CPL; ++j) t[j] = 0.0f;
      }
      if constexpr (k_first) kacc = 0.0f;
      kacc = fmaf(tm.c, Y[tm.mu2], kacc);
      if constexpr (k_last) {
#pragma unroll
        for (int j = 0; j < Cfg::CPL; ++j) t[j] = fmaf(kacc, xv[j][tm.mu1], t[j]);
      }
      if constexpr (pm_last) {
#pragma unroll
        for (int j = 0; j < Cfg::CPL; ++j) acc[j][tm.mu3] = fmaf(we[j], t[j], acc[j][tm.mu3]);
      }
    });
  }
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int L, int PS, int C, bool RADIAL, bool ATOMIC, bool XB, bool OB = false>
__global__ __launch_bounds__(EdgeCfg<C>::THREADS) void conv_edge_kernel(
    int N, int E, const int* __restrict__ row_ptr, const float* __restrict__ vec, const int* __restrict__ src,
    const int* __restrict__ dst, const typename EdgeMsg<L, PS, C, RADIAL, XB>::XT* __restrict__ x,
    const float* __restrict__ w, float* __restrict__ out, float inv_rc) {
  using Cfg = EdgeCfg<C>;
  using T = Tables<L, PS>;
  using M = EdgeMsg<L, PS, C, RADIAL, XB>;
  constexpr int K = num_comp(L);
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int g = lane / Cfg::CL;
  const int cl = lane % Cfg::CL;

  float wreg[Cfg::CPL][T::P];
  if constexpr (!RADIAL) {
#pragma unroll
    for (int j = 0; j < Cfg::CPL; ++j)
#pragma unroll
      for (int p = 0; p < T::P; ++p) wreg[j][p] = w[p * C + cl + j * Cfg::CL];
  }

  float acc[Cfg::CPL][K];
  if constexpr (!ATOMIC) {
    const int row = blockIdx.x * Cfg::WAVES + wv;
    if (row >= N) return;
    int e_beg = 0, e_end = 0;
    if (E > 0) {
      e_beg = min(max(row_ptr[row], 0), E);
      e_end = min(max(row_ptr[row + 1], e_beg), E);
    }
#pragma unroll
    for (int j = 0; j < Cfg::CPL; ++j)
#pragma unroll
      for (int k = 0; k < K; ++k) acc[j][k] = 0.0f;
    for (int e = e_beg + g; e < e_end; e += Cfg::G) M::run(e, N, cl, vec, src, x, w, wreg, inv_rc, acc);
    // combine the lane groups (lanes cl, cl + CL, cl + 2 CL, ...)
#pragma unroll
    for (int off = Cfg::CL; off < kWave; off <<= 1)
#pragma unroll
      for (int j = 0; j < Cfg::CPL; ++j)
#pragma unroll
        for (int k = 0; k < K; ++k) acc[j][k] += __shfl_xor(acc[j][k], off);
    if (g == 0) {
#pragma unroll
      for (int j = 0; j < Cfg::CPL; ++j) {
        float* op = out + ((size_t)row * C + cl + j * Cfg::CL) * K;
        if constexpr (K % 4 == 0) {
#pragma unroll
          for (int q = 0; q < K / 4; ++q)
            reinterpret_cast<f4*>(op)[q] = f4{acc[j][4 * q], acc[j][4 * q + 1], acc[j][4 * q + 2], acc[j][4 * q + 3]};
        } else {
#pragma unroll
          for (int k = 0; k < K; ++k) op[k] = acc[j][k];
        }
      }
    }
  } else {
    // The wave's G messages (G*C*K = 64*CPL*K floats, one contiguous C*K
    // block per edge) go through LDS so that atomic instruction i covers
    // floats 64i .. 64i+63: 256 contiguous bytes (two cache lines) instead of
    // one float per 64-byte channel row.
    constexpr int MSG = C * K;               // floats per edge message
    constexpr int NI = Cfg::CPL * K;         // atomic instructions per wave and round
    __shared__ float xch[Cfg::WAVES][kWave * NI];
    __shared__ int xdst[Cfg::WAVES][Cfg::G];
    float* const xw = xch[wv];
    const long long base = ((long long)blockIdx.x * Cfg::WAVES + wv) * Cfg::EPW;
    const int e_end = (int)min((long long)E, base + Cfg::EPW);
    for (int e0 = (int)base; e0 < e_end; e0 += Cfg::G) {  // wave-uniform rounds of G edges
      const int e = e0 + g;
      const bool valid = e < e_end;
#pragma unroll
      for (int j = 0; j < Cfg::CPL; ++j)
#pragma unroll
        for (int k = 0; k < K; ++k) acc[j][k] = 0.0f;
      if (valid) M::run(e, N, cl, vec, src, x, w, wreg, inv_rc, acc);
#pragma unroll
      for (int j = 0; j < Cfg::CPL; ++j)
#pragma unroll
        for (int k = 0; k < K; ++k) xw[(g * C + cl + j * Cfg::CL) * K + k] = acc[j][k];
      if (cl == 0) xdst[wv][g] = valid ? clamp_index(dst[e], N) : -1;  // -1: no edge in this slot
      wave_lds_sync();
      if constexpr (OB) {
        // lane pairs of consecutive floats (MSG is even, so a pair never straddles two messages): one
        // packed atomic covers 4 bytes of out, an instruction 256 contiguous bytes
        constexpr int NPAIR = kWave * NI / 2;
        bf16x2_t* const ob = reinterpret_cast<bf16x2_t*>(out);
#pragma unroll
        for (int i = 0; i < (NPAIR + kWave - 1) / kWave; ++i) {
          const int pr = kWave * i + lane;
          if (pr < NPAIR) {
            const int f = 2 * pr;
            const int d = xdst[wv][f / MSG];
            if (d >= 0) {
              const bf16x2_t v = {to_bf16(xw[f]), to_bf16(xw[f + 1])};
              __builtin_amdgcn_global_atomic_fadd_v2bf16(
                  (__attribute__((address_space(1))) bf16x2_t*)(ob + ((size_t)d * MSG + f % MSG) / 2), v);
            }
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int f = kWave * i + lane;      // float index in the wave's messages
          const int d = xdst[wv][f / MSG];
          if (d >= 0) unsafeAtomicAdd(out + (size_t)d * MSG + f % MSG, xw[f]);  // hardware fp32 atomic
        }
      }
      wave_lds_sync();
    }
  }
}

// Per-edge messages without the destination sum (the page's fused kernel
// output, section "3. operator fusion"): msg[e, c, :] for every edge, lane =
// channel; a wave's store of one edge covers its C*K*4 contiguous bytes.
template <int L, int PS, int C, bool RADIAL>
__global__ __launch_bounds__(EdgeCfg<C>::THREADS) void conv_msg_kernel(int N, int E, const float* __restrict__ vec,
                                                                       const int* __restrict__ src,
                                                                       const float* __restrict__ x,
                                                                       const float* __restrict__ w,
                                                                       float* __restrict__ msg, float inv_rc) {
  using Cfg = EdgeCfg<C>;
  using T = Tables<L, PS>;
  using M = EdgeMsg<L, PS, C, RADIAL>;
  constexpr int K = num_comp(L);
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int g = lane / Cfg::CL;
  const int cl = lane % Cfg::CL;
  float wreg[Cfg::CPL][T::P];
  if constexpr (!RADIAL) {
#pragma unroll
    for (int j = 0; j < Cfg::CPL; ++j)
#pragma unroll
      for (int p = 0; p < T::P; ++p) wreg[j][p] = w[p * C + cl + j * Cfg::CL];
  }
  const long long base = ((long long)blockIdx.x * Cfg::WAVES + wv) * Cfg::EPW;
  const int e_end = (int)min((long long)E, base + Cfg::EPW);
  for (int e = (int)base + g; e < e_end; e += Cfg::G) {
    float acc[Cfg::CPL][K];
#pragma unroll
    for (int j = 0; j < Cfg::CPL; ++j)
#pragma unroll
      for (int k = 0; k < K; ++k) acc[j][k] = 0.0f;
    M::run(e, N, cl, vec, src, x, w, wreg, inv_rc, acc);
#pragma unroll
    for (int j = 0; j < Cfg::CPL; ++j) {
      float* op = msg + ((size_t)e * C + cl + j * Cfg::CL) * K;
      if constexpr (K % 4 == 0) {
#pragma unroll
        for (int q = 0; q < K / 4; ++q)
          reinterpret_cast<f4*>(op)[q] = f4{acc[j][4 * q], acc[j][4 * q + 1], acc[j][4 * q + 2], acc[j][4 * q + 3]};
      } else {
#pragma unroll
        for (int k = 0; k < K; ++k) op[k] = acc[j][k];
      }
    }
  }
}

template <int L, int PS, int C, bool RADIAL>
static hipError_t launch_msg_t(const ConvArgs& a) {
  using Cfg = EdgeCfg<C>;
  if (a.E == 0) return hipSuccess;
  const long long per_block = (long long)Cfg::WAVES * Cfg::EPW;
  const unsigned blocks = (unsigned)((a.E + per_block - 1) / per_block);
  hipLaunchKernelGGL((conv_msg_kernel<L, PS, C, RADIAL>), dim3(blocks), dim3(Cfg::THREADS), 0, a.stream, (int)a.N,
                     (int)a.E, a.vec, a.src, a.x, a.w, a.out, RADIAL ? 1.0f / a.r_cut : 0.0f);
  return hipGetLastError();
}

template <int L, int PS>
static hipError_t dispatch_msg_c(const ConvArgs& a) {
  const bool radial = a.weight_mode == 1;
  switch (a.C) {
    case 8: return radial ? launch_msg_t<L, PS, 8, true>(a) : launch_msg_t<L, PS, 8, false>(a);
    case 16: return radial ? launch_msg_t<L, PS, 16, true>(a) : launch_msg_t<L, PS, 16, false>(a);
    case 32: return radial ? launch_msg_t<L, PS, 32, true>(a) : launch_msg_t<L, PS, 32, false>(a);
    case 64: return radial ? launch_msg_t<L, PS, 64, true>(a) : launch_msg_t<L, PS, 64, false>(a);
    case 128: return radial ? launch_msg_t<L, PS, 128, true>(a) : launch_msg_t<L, PS, 128, false>(a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_conv_messages(const ConvArgs& a) {
  switch (a.lmax * 2 + a.path_set) {
    case 0: return dispatch_msg_c<0, 0>(a);
    case 1: return dispatch_msg_c<0, 1>(a);
    case 2: return dispatch_msg_c<1, 0>(a);
    case 3: return dispatch_msg_c<1, 1>(a);
    case 4: return dispatch_msg_c<2, 0>(a);
    case 5: return dispatch_msg_c<2, 1>(a);
    case 6: return dispatch_msg_c<3, 0>(a);
    case 7: return dispatch_msg_c<3, 1>(a);
    default: return hipErrorInvalidValue;
  }
}

// Test-only twin of the sorted walk: same launch shape, row -> wave and
// edge -> lane-group dealing, and the same cross-lane combine.
template <int C>
__global__ __launch_bounds__(EdgeCfg<C>::THREADS) void probe_edge_kernel(int N, int E,
                                                                        const int* __restrict__ row_ptr,
                                                                        const int* __restrict__ src,
                                                                        int* __restrict__ count,
                                                                        long long* __restrict__ src_sum) {
  using Cfg = EdgeCfg<C>;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int g = lane / Cfg::CL;
  const int cl = lane % Cfg::CL;
  const int row = blockIdx.x * Cfg::WAVES + wv;
  if (row >= N) return;
  int e_beg = 0, e_end = 0;
  if (E > 0) {
    e_beg = min(max(row_ptr[row], 0), E);
    e_end = min(max(row_ptr[row + 1], e_beg), E);
  }
  int cnt = 0;
  long long sum = 0;
  for (int e = e_beg + g; e < e_end; e += Cfg::G) {
    if (cl == 0) {
      cnt += 1;
      sum += clamp_index(src[e], N);
    }
  }
  for (int off = Cfg::CL; off < kWave; off <<= 1) {
    cnt += __shfl_xor(cnt, off);
    sum += __shfl_xor(sum, off);
  }
  if (lane == 0) {
    count[row] = cnt;
    src_sum[row] = sum;
  }
}

template <int L, int PS, int C, bool RADIAL, bool ATOMIC, bool XB, bool OB = false>
static hipError_t launch_edge_t(const ConvArgs& a) {
  using Cfg = EdgeCfg<C>;
  using XT = typename EdgeMsg<L, PS, C, RADIAL, XB>::XT;
  const XT* x = reinterpret_cast<const XT*>(a.x);
  const float inv_rc = RADIAL ? 1.0f / a.r_cut : 0.0f;
  if constexpr (ATOMIC) {
    if (a.N > 0) {  // zero bits are 0.0 in either type; a bf16 out is N C K / 2 floats (C is even)
      hipError_t err = launch_fill_zero(a.out, a.N * a.C * num_comp(L) / (OB ? 2 : 1), a.stream);
      if (err != hipSuccess) return err;
    }
    if (a.E == 0) return hipSuccess;
    const long long per_block = (long long)Cfg::WAVES * Cfg::EPW;
    const unsigned blocks = (unsigned)((a.E + per_block - 1) / per_block);
    hipLaunchKernelGGL((conv_edge_kernel<L, PS, C, RADIAL, true, XB, OB>), dim3(blocks), dim3(Cfg::THREADS), 0,
                       a.stream, (int)a.N, (int)a.E, a.row_ptr, a.vec, a.src, a.dst, x, a.w, a.out, inv_rc);
  } else {
    if (a.N == 0) return hipSuccess;
    const unsigned blocks = (unsigned)((a.N + Cfg::WAVES - 1) / Cfg::WAVES);
    hipLaunchKernelGGL((conv_edge_kernel<L, PS, C, RADIAL, false, XB>), dim3(blocks), dim3(Cfg::THREADS), 0,
                       a.stream, (int)a.N, (int)a.E, a.row_ptr, a.vec, a.src, a.dst, x, a.w, a.out, inv_rc);
  }
  return hipGetLastError();
}

template <int L, int PS, int C, bool XB>
static hipError_t dispatch_edge_mode_x(const ConvArgs& a) {
  const bool radial = a.weight_mode == 1, atomic = a.edge_order == 1;
  if (atomic && a.out_bf16)
    return radial ? launch_edge_t<L, PS, C, true, true, XB, true>(a) : launch_edge_t<L, PS, C, false, true, XB, true>(a);
  if (radial)
    return atomic ? launch_edge_t<L, PS, C, true, true, XB>(a) : launch_edge_t<L, PS, C, true, false, XB>(a);
  return atomic ? launch_edge_t<L, PS, C, false, true, XB>(a) : launch_edge_t<L, PS, C, false, false, XB>(a);
}

template <int L, int PS, int C>
static hipError_t dispatch_edge_mode(const ConvArgs& a) {
  return a.x_bf16 ? dispatch_edge_mode_x<L, PS, C, true>(a) : dispatch_edge_mode_x<L, PS, C, false>(a);
}

template <int L, int PS>
static hipError_t dispatch_edge_c(const ConvArgs& a) {
  switch (a.C) {
    case 8: return dispatch_edge_mode<L, PS, 8>(a);
    case 16: return dispatch_edge_mode<L, PS, 16>(a);
    case 32: return dispatch_edge_mode<L, PS, 32>(a);
    case 64: return dispatch_edge_mode<L, PS, 64>(a);
    case 128: return dispatch_edge_mode<L, PS, 128>(a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_conv_edge(const ConvArgs& a) {
  switch (a.lmax * 2 + a.path_set) {
    case 0: return dispatch_edge_c<0, 0>(a);
    case 1: return dispatch_edge_c<0, 1>(a);
    case 2: return dispatch_edge_c<1, 0>(a);
    case 3: return dispatch_edge_c<1, 1>(a);
    case 4: return dispatch_edge_c<2, 0>(a);
    case 5: return dispatch_edge_c<2, 1>(a);
    case 6: return dispatch_edge_c<3, 0>(a);
    case 7: return dispatch_edge_c<3, 1>(a);
    default: return hipErrorInvalidValue;
  }
}

template <int C>
static hipError_t launch_probe_edge_t(const ProbeArgs& a) {
  using Cfg = EdgeCfg<C>;
  if (a.N == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((a.N + Cfg::WAVES - 1) / Cfg::WAVES);
  hipLaunchKernelGGL((probe_edge_kernel<C>), dim3(blocks), dim3(Cfg::THREADS), 0, a.stream, (int)a.N, (int)a.E,
                     a.row_ptr, a.src, a.count, a.src_sum);
  return hipGetLastError();
}

hipError_t launch_probe_edge(const ProbeArgs& a) {
  switch (a.C) {
    case 8: return launch_probe_edge_t<8>(a);
    case 16: return launch_probe_edge_t<16>(a);
    case 32: return launch_probe_edge_t<32>(a);
    case 64: return launch_probe_edge_t<64>(a);
    case 128: return launch_probe_edge_t<128>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace eqtp
