// conv_node.hip -- fused convolution for dst-sorted edges with fixed path
// weights, factored per destination node and run on the fp32 matrix cores.
//
// What is computed (Batmobile page, sections "2. register intermediate
// computation" and "3. operator fusion"): for every destination node n
//   out[n,c,mu3] = sum_e sum_p w[p,c] sum_{mu1,mu2} C^p[mu1,mu2,mu3] x[src_e,c,mu1] Y_mu2(vec_e).
// Because the weights do not depend on the edge and the product is bilinear,
// the edge sum can be taken first:
//   G_n[c,mu1,mu2] = sum_{e in row n} x[src_e,c,mu1] * Y_mu2(vec_e)
//   out[n,c,mu3]   = sum_p w[p,c] sum_{mu1,mu2} C^p[mu1,mu2,mu3] G_n[c,mu1,mu2].
// G_n is a dense [K x K] outer-product sum per channel -- a K-deep contraction
// over the row's edges that maps onto v_mfma_f32_16x16x4_f32 (rows mu2,
// columns = 16 channels, 4 edges per instruction).  The coupling then runs
// once per node instead of once per edge, with the coefficients folded into
// the instruction stream.  Messages never exist in memory.
//
// Work decomposition (one workgroup per destination row):
//   * NW = max(1, C/16) waves; wave w accumulates G for channels 16w..16w+15.
//   * The row's edges are staged 64 at a time: lane i loads edge i's vector
//     and source index (coalesced), evaluates its harmonics and writes them to
//     the wave's LDS staging area.
//   * Each 4-edge step: lane l feeds A = Y[edge l/16][mu2 = l%16] and, for
//     each mu1, B = x[src(edge l/16), channel 16w + l%16, mu1] from one
//     contiguous K-float load per lane.
//   * After the row, G goes to LDS; every wave then contracts one group of
//     output components for C lanes = C channels, reading G rows with an odd
//     stride (no bank conflicts), and the output tile is stored coalesced.
#include "eqtp_device.hpp"
#include "eqtp_kernels.hpp"

namespace eqtp {

template <int L, int C>
struct NodeCfg {
  static constexpr int K = num_comp(L);
  static constexpr int NW = C >= 16 ? C / 16 : 1;        // waves per workgroup
  static constexpr int CW = C >= 16 ? 16 : C;            // channels per wave
  static constexpr int GS = (K * K) % 2 ? K * K : K * K + 1;  // LDS floats per channel (odd)
  static constexpr int SLICE = CW * GS;                  // LDS floats per wave's G slice
  static constexpr int STG = 64 * 16 + 64;               // staging: Y[64][16] + src[64]
  static constexpr bool STG_IN_SLICE = SLICE >= STG;
  static constexpr int LDS = NW * SLICE + (STG_IN_SLICE ? 0 : NW * STG);
  static constexpr int CB = C > 64 ? C / 64 : 1;         // 64-channel blocks in the epilogue
  static constexpr int NG = NW / CB;                     // output-component groups
  static constexpr int THREADS = NW * kWave;
  static_assert(C * K <= LDS, "output tile must fit in LDS");
  static_assert(LDS * 4 <= 160 * 1024, "LDS budget");
};

// One row -> wave -> lane -> step walk.  Calls stage(cb, cnt) once per chunk
// of up to 64 edges; for every 4-edge step of the chunk, load(el) issues the
// step's memory reads (el = this lane's edge slot 0..63 in the staging area)
// and compute(data) consumes them.  Loads run one step ahead of compute.
template <class Stage, class Load, class Compute>
__device__ __forceinline__ void node_row_walk(int e_beg, int e_end, Stage&& stage, Load&& load, Compute&& compute) {
  const int lane = threadIdx.x & 63;
  const int kq = lane >> 4;
  for (int cb = e_beg; cb < e_end; cb += 64) {
    const int cnt = min(64, e_end - cb);
    stage(cb, cnt);
    wave_lds_sync();
    const int nsteps = (cnt + 3) >> 2;
    auto cur = load(kq);
    for (int st = 0; st < nsteps; ++st) {
      decltype(cur) nxt = cur;
      if (st + 1 < nsteps) nxt = load((st + 1) * 4 + kq);
      compute(cur);
      cur = nxt;
    }
    wave_lds_sync();
  }
}

template <int L, int PS, int C>
__global__ __launch_bounds__((NodeCfg<L, C>::THREADS)) void conv_node_kernel(int N, int E,
                                                                           const int* __restrict__ row_ptr,
                                                                           const float* __restrict__ vec,
                                                                           const int* __restrict__ src,
                                                                           const float* __restrict__ x,
                                                                           const float* __restrict__ w,
                                                                           float* __restrict__ out) {
  using Cfg = NodeCfg<L, C>;
  using T = Tables<L, PS>;
  constexpr int K = Cfg::K;
  __shared__ __attribute__((aligned(16))) float lds[Cfg::LDS];

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int row = blockIdx.x;
  int e_beg = 0, e_end = 0;
  if (E > 0) {
    e_beg = min(max(row_ptr[row], 0), E);
    e_end = min(max(row_ptr[row + 1], e_beg), E);
  }

  float* slice = lds + wv * Cfg::SLICE;
  float* ystg = Cfg::STG_IN_SLICE ? slice : lds + Cfg::NW * Cfg::SLICE + wv * Cfg::STG;
  int* sstg = reinterpret_cast<int*>(ystg + 64 * 16);

  const int cl = lane & 15;                  // column of the MFMA tile = channel within the wave
  const bool c_ok = cl < Cfg::CW;
  const int c_load = wv * Cfg::CW + (c_ok ? cl : 0);

  f4 acc[K];
#pragma unroll
  for (int k = 0; k < K; ++k) acc[k] = f4{0.f, 0.f, 0.f, 0.f};

  auto stage = [&](int cb, int cnt) {
    const bool valid = lane < cnt;
    const int e = cb + (valid ? lane : 0);
    const float vx = vec[3 * e + 0], vy = vec[3 * e + 1], vz = vec[3 * e + 2];
    const int s = clamp_index(src[e], N);
    float Y[16];
    sh_eval<L>(vx, vy, vz, Y);
    const float m = valid ? 1.0f : 0.0f;  // padding slots contribute nothing
    f4* yd = reinterpret_cast<f4*>(ystg + lane * 16);
#pragma unroll
    for (int q = 0; q < 4; ++q) yd[q] = f4{m * Y[4 * q], m * Y[4 * q + 1], m * Y[4 * q + 2], m * Y[4 * q + 3]};
    sstg[lane] = s;
  };

  struct StepData {
    float a;
    float xv[K];
  };
  auto load = [&](int el) {
    StepData d;
    d.a = ystg[el * 16 + cl];
    const int s = sstg[el];
    const float* xp = x + ((size_t)s * C + c_load) * K;
    if constexpr (K % 4 == 0) {
#pragma unroll
      for (int q = 0; q < K / 4; ++q) {
        const f4 t = c_ok ? reinterpret_cast<const f4*>(xp)[q] : f4{0.f, 0.f, 0.f, 0.f};
        d.xv[4 * q] = t[0];
        d.xv[4 * q + 1] = t[1];
        d.xv[4 * q + 2] = t[2];
        d.xv[4 * q + 3] = t[3];
      }
    } else {
#pragma unroll
      for (int k = 0; k < K; ++k) d.xv[k] = c_ok ? xp[k] : 0.0f;
    }
    return d;
  };
  auto compute = [&](const StepData& d) {
#pragma unroll
    for (int k = 0; k < K; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x4f32(d.a, d.xv[k], acc[k], 0, 0, 0);
  };

  node_row_walk(e_beg, e_end, stage, load, compute);

  // G[c][mu1][mu2] -> LDS.  Lane l holds G[16w + l%16][mu1][mu2 = 4(l/16) + v].
  if (c_ok) {
    float* gc = slice + cl * Cfg::GS;
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int mu2 = 4 * (lane >> 4) + v;
        if (mu2 < K) gc[k * K + mu2] = acc[k][v];
      }
  }
  __syncthreads();

  // Epilogue: wave -> (64-channel block, output-component group); lane = channel.
  const int cblk = wv % Cfg::CB;
  const int grp = wv / Cfg::CB;
  const int c = cblk * 64 + lane;
  float ov[K];
#pragma unroll
  for (int k = 0; k < K; ++k) ov[k] = 0.0f;
  if (c < C) {
    const float* gc = lds + c * Cfg::GS;
    float wr[T::P];
#pragma unroll
    for (int p = 0; p < T::P; ++p) wr[p] = w[p * C + c];
    static_for<0, Cfg::NG>([&](auto gi) {
      constexpr int G = decltype(gi)::value;
      constexpr int TB = term_begin_for_mu3<L, PS>(group_mu3_begin<L, PS>(Cfg::NG, G));
      constexpr int TE = term_begin_for_mu3<L, PS>(group_mu3_begin<L, PS>(Cfg::NG, G + 1));
      if (grp == G) {
        float t = 0.0f;
        static_for<TB, TE>([&](auto ii) {
          constexpr int i = decltype(ii)::value;
          constexpr eqtp_gen::CgTerm tm = T::by_out[i];
          constexpr bool first = (i == TB) || T::by_out[i - 1].p != tm.p || T::by_out[i - 1].mu3 != tm.mu3;
          constexpr bool last = (i + 1 == TE) || T::by_out[i + 1].p != tm.p || T::by_out[i + 1].mu3 != tm.mu3;
          const float g = gc[tm.mu1 * K + tm.mu2];
          t = first ? tm.c * g : fmaf(tm.c, g, t);
          if constexpr (last) ov[tm.mu3] = fmaf(wr[tm.p], t, ov[tm.mu3]);
        });
      }
    });
  }
  __syncthreads();
  // Output tile [C][K] in LDS (this wave's component group only), then a
  // coalesced store of the row.
  if (c < C) {
    static_for<0, Cfg::NG>([&](auto gi) {
      constexpr int G = decltype(gi)::value;
      constexpr int MB = group_mu3_begin<L, PS>(Cfg::NG, G);
      constexpr int ME = group_mu3_begin<L, PS>(Cfg::NG, G + 1);
      if (grp == G) {
#pragma unroll
        for (int k = MB; k < ME; ++k) lds[c * K + k] = ov[k];
      }
    });
  }
  __syncthreads();
  f4* orow = reinterpret_cast<f4*>(out + (size_t)row * C * K);
  const f4* trow = reinterpret_cast<const f4*>(lds);
  for (int i = threadIdx.x; i < C * K / 4; i += Cfg::THREADS) orow[i] = trow[i];
}

// Test-only twin of the walk above: the same launch shape, staging and step
// schedule, counting edges and summing source indices per row.
template <int L, int C>
__global__ __launch_bounds__((NodeCfg<L, C>::THREADS)) void probe_node_kernel(int N, int E,
                                                                            const int* __restrict__ row_ptr,
                                                                            const int* __restrict__ src,
                                                                            int* __restrict__ count,
                                                                            long long* __restrict__ src_sum) {
  using Cfg = NodeCfg<L, C>;
  __shared__ __attribute__((aligned(16))) float lds[Cfg::LDS];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int row = blockIdx.x;
  int e_beg = 0, e_end = 0;
  if (E > 0) {
    e_beg = min(max(row_ptr[row], 0), E);
    e_end = min(max(row_ptr[row + 1], e_beg), E);
  }
  float* slice = lds + wv * Cfg::SLICE;
  float* ystg = Cfg::STG_IN_SLICE ? slice : lds + Cfg::NW * Cfg::SLICE + wv * Cfg::STG;
  int* sstg = reinterpret_cast<int*>(ystg + 64 * 16);
  int cnt_acc = 0;
  long long sum_acc = 0;
  auto stage = [&](int cb, int cnt) {
    const bool valid = lane < cnt;
    const int e = cb + (valid ? lane : 0);
    ystg[lane * 16] = valid ? 1.0f : 0.0f;  // the "harmonic" flags real slots
    sstg[lane] = clamp_index(src[e], N);
  };
  struct StepData {
    bool real;
    int s;
  };
  auto load = [&](int el) { return StepData{ystg[el * 16] != 0.0f, sstg[el]}; };
  auto compute = [&](const StepData& d) {
    if ((lane & 15) == 0 && d.real) {
      cnt_acc += 1;
      sum_acc += d.s;
    }
  };
  node_row_walk(e_beg, e_end, stage, load, compute);
  // lanes 0, 16, 32, 48 hold partial results; fold them
  for (int off = 16; off < 64; off <<= 1) {
    cnt_acc += __shfl_xor(cnt_acc, off);
    sum_acc += __shfl_xor(sum_acc, off);
  }
  if (wv == 0 && lane == 0) {
    count[row] = cnt_acc;
    src_sum[row] = sum_acc;
  }
}

template <int L, int PS, int C>
static hipError_t launch_node(const ConvArgs& a) {
  using Cfg = NodeCfg<L, C>;
  if (a.N == 0) return hipSuccess;
  hipLaunchKernelGGL((conv_node_kernel<L, PS, C>), dim3((unsigned)a.N), dim3(Cfg::THREADS), 0, a.stream, (int)a.N,
                     (int)a.E, a.row_ptr, a.vec, a.src, a.x, a.w, a.out);
  return hipGetLastError();
}

template <int L, int C>
static hipError_t launch_probe_node(const ProbeArgs& a) {
  using Cfg = NodeCfg<L, C>;
  if (a.N == 0) return hipSuccess;
  hipLaunchKernelGGL((probe_node_kernel<L, C>), dim3((unsigned)a.N), dim3(Cfg::THREADS), 0, a.stream, (int)a.N,
                     (int)a.E, a.row_ptr, a.src, a.count, a.src_sum);
  return hipGetLastError();
}

#define EQTP_C_SWITCH(C_, BODY) \
  switch (C_) {                 \
    case 8: { constexpr int CC = 8; BODY; } \
    case 16: { constexpr int CC = 16; BODY; } \
    case 32: { constexpr int CC = 32; BODY; } \
    case 64: { constexpr int CC = 64; BODY; } \
    case 128: { constexpr int CC = 128; BODY; } \
    default: return hipErrorInvalidValue; \
  }

template <int L, int PS>
static hipError_t dispatch_node_c(const ConvArgs& a) {
  EQTP_C_SWITCH(a.C, return (launch_node<L, PS, CC>(a)))
}

hipError_t launch_conv_node(const ConvArgs& a) {
  const int key = a.lmax * 2 + a.path_set;
  switch (key) {
    case 0: return dispatch_node_c<0, 0>(a);
    case 1: return dispatch_node_c<0, 1>(a);
    case 2: return dispatch_node_c<1, 0>(a);
    case 3: return dispatch_node_c<1, 1>(a);
    case 4: return dispatch_node_c<2, 0>(a);
    case 5: return dispatch_node_c<2, 1>(a);
    case 6: return dispatch_node_c<3, 0>(a);
    case 7: return dispatch_node_c<3, 1>(a);
    default: return hipErrorInvalidValue;
  }
}

template <int L>
static hipError_t dispatch_probe_node_c(const ProbeArgs& a) {
  EQTP_C_SWITCH(a.C, return (launch_probe_node<L, CC>(a)))
}

hipError_t launch_probe_node(const ProbeArgs& a) {
  switch (a.lmax) {
    case 0: return dispatch_probe_node_c<0>(a);
    case 1: return dispatch_probe_node_c<1>(a);
    case 2: return dispatch_probe_node_c<2>(a);
    case 3: return dispatch_probe_node_c<3>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace eqtp
