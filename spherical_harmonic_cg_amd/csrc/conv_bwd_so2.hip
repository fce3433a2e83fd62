// conv_bwd_so2.hip -- gradients of the fixed-weight convolution in the
// edge-aligned (SO(2)) form, for lmax 0..6 (E2Former-V2 page, section 2.1
// "derivation of EAAS"; the page names a PyTorch autograd function with a
// backward as the integration path, section "extension possibilities").
//
// For L = sum grad_out * out with out[d] = sum_{e: dst_e = d} D^T P_w(D x[src_e])
// (D = D(R_e) the action on the real harmonics of the rotation R_e that takes
// the edge direction to the z axis, P_w the coupling with the harmonics of the
// z axis and per-path weights w[p, c]; see conv_so2.hip), per edge and
// channel, with x' = D x[src_e] and g' = D grad_out[dst_e] in the edge frame:
//   grad_x[src_e] += D^T v',          v' = P_w^T g'
//   grad_w[p, c]  += g' . P_p x'      (P_p: path p's part of the coupling)
// and for the edge vector: dL/dvec = sum_mu dL/dY_mu dY_mu/dvec.  At the z
// axis only the m = +-1 harmonics have a tangential derivative, and
//   dY(z)/dx = L_y Y(z),   dY(z)/dy = -L_x Y(z)
// with L_a the generator of rotations about axis a (L_a = d/de D(R_a(e)) at
// e = 0).  The coupling is invariant under rotations, so for every generator
//   C(L a, Y, b) + C(a, L Y, b) + C(a, Y, L b) = 0,
// which moves the derivative off the harmonics onto x' and g':
//   G_x = -(v' . L_y x' + u' . L_y g'),   G_y = v' . L_x x' + u' . L_x g',
//   dL/dvec = R_e^T (G_x, G_y, 0) / |vec|        (summed over channels),
// with u' = P_w x' the message in the frame.  So the whole gradient costs two
// rotations in, one walk of the sparse coupling (624 terms at lmax 6, not the
// 6460 of the full coupling), four products with the 72-entry generators
// and one rotation back.  A zero edge vector drops the paths with l2 > 0 (as
// the forward does) and has grad_vec = 0.  L_x, L_y and the identity above
// are generated and checked in gen_so2_table.py.
//
// Lane mapping as in the forward: lane = channel (C <= 64: 64/C edges per
// wave round; C = 128: two channels per lane).  Persistent waves take
// destination rows (dst-sorted edges), runs of edges (any order, dst[]) or
// source rows (edges grouped by source: grad_x summed per row, no atomics).
// grad_x: fp32 atomics after an LDS exchange (each instruction adds 64
// consecutive floats of one source's row); grad_w: per-lane sums in
// registers over all of the wave's edges, then LDS atomics into the
// workgroup's [P][C] sums and one add to memory per workgroup; grad_vec: the
// channel sum by xor shuffles, one store per edge.
#include "eqtp_device.hpp"
#include "eqtp_kernels.hpp"
#include "so2_device.hpp"

namespace eqtp {

template <int L, int PS, int C>
struct So2BwdCfg {
  static constexpr int K = num_comp(L);
  static constexpr int P = So2Tables<L, PS>::P;
  static constexpr int CPL = C > 64 ? C / 64 : 1;  // channels per lane
  static constexpr int CL = C / CPL;               // lanes per edge group
  static constexpr int G = kWave / CL;             // edge groups per wave
  static constexpr int EPW = 8 * G;                // edges per task, any order
  // grad_w sums over the wave's edges: per-lane registers when there are few
  // of them, else lane-private LDS slots (a plain read-add-write per path and
  // edge: LDS float atomics there cost far more)
  static constexpr bool GW_REG = P * CPL <= 34;
  static constexpr int64_t lds_bytes(int waves, bool wl) {
    return 4LL * ((GW_REG ? (int64_t)P * C : (int64_t)waves * P * kWave * CPL) +  // grad_w sums
                  (int64_t)waves * kWave * CPL * K +                             // grad_x exchange
                  (wl ? (int64_t)P * C : 0) + waves * G);                        // weights, sources
  }
  static constexpr int64_t kLds = 160 * 1024;
  // waves per workgroup: as many as fit (up to 4) without the weights in LDS;
  // the weights are staged there too if they still fit, else read through the caches
  static constexpr int WAVES = lds_bytes(4, false) <= kLds ? 4 : lds_bytes(3, false) <= kLds ? 3
                             : lds_bytes(2, false) <= kLds ? 2 : 1;
  static constexpr bool WL_LDS = lds_bytes(WAVES, true) <= kLds;
  static constexpr int64_t LDS = lds_bytes(WAVES, WL_LDS);
  static constexpr int PER_CU = LDS * 2 <= kLds ? 2 : 1;  // workgroups per compute unit
  static constexpr int THREADS = WAVES * kWave;
  static_assert(LDS <= kLds, "LDS budget");
};

template <int K>
__device__ __forceinline__ void load_vec(const float* __restrict__ p, float (&v)[K]) {
  if constexpr (K % 4 == 0) {
#pragma unroll
    for (int q = 0; q < K / 4; ++q) {
      const f4 t4 = reinterpret_cast<const f4*>(p)[q];
      v[4 * q] = t4[0];
      v[4 * q + 1] = t4[1];
      v[4 * q + 2] = t4[2];
      v[4 * q + 3] = t4[3];
    }
  } else {
#pragma unroll
    for (int k = 0; k < K; ++k) v[k] = p[k];
  }
}

// the path of the first term after path p's terms (which start at term i), or -1
template <class T>
constexpr int next_path_after(int i) {
  for (int k = i; k < T::NT; ++k)
    if (T::terms[k].p != T::terms[i].p) return T::terms[k].p;
  return -1;
}

// mode 0: edges in any order (runs of EPW edges; src, dst per edge); 1: dst-sorted (row_ptr over
// destinations, src per edge); 2: grouped by source (row_ptr over sources, dst per edge, perm[i] = the
// input index of grouped edge i for grad_vec): grad_x is summed per source row in the wave's LDS and
// written once, no atomics.  ntasks: rows (modes 1, 2) or runs.
template <int L, int PS, int C>
constexpr int kBwdSo2Threads = So2BwdCfg<L, PS, C>::THREADS;
template <int L, int PS, int C>  // waves per SIMD that the LDS allows (the register budget follows)
constexpr int kBwdSo2Occ = So2BwdCfg<L, PS, C>::WAVES * So2BwdCfg<L, PS, C>::PER_CU >= 8 ? 2 : 1;

// CT: channels per node row of x, grad_out and grad_x and per path row of w and grad_w (C, or 128 when a
// C = 128 problem runs as two 64-channel halves, the pointers then offset to the half's first channel);
// GV_ADD: grad_vec adds to what the first half wrote instead of storing
template <int L, int PS, int C, int CT = C, bool GV_ADD = false>
__global__ __launch_bounds__((kBwdSo2Threads<L, PS, C>)) __attribute__((amdgpu_waves_per_eu(
    kBwdSo2Occ<L, PS, C>))) void conv_bwd_so2_kernel(
    int N, int E, long long ntasks, int mode, const int* __restrict__ row_ptr, const float* __restrict__ vec,
    const int* __restrict__ src, const int* __restrict__ dst, const int* __restrict__ perm,
    const float* __restrict__ x, const float* __restrict__ w, const float* __restrict__ gout, float* __restrict__ gx,
    float* __restrict__ gw, float* __restrict__ gvec) {
  using Cfg = So2BwdCfg<L, PS, C>;
  using T = So2Tables<L, PS>;
  constexpr int K = num_comp(L);
  constexpr int MSG = C * K;        // floats of one source row
  constexpr int NI = Cfg::CPL * K;  // floats per lane of one round's grad_x rows
  constexpr int GWS = Cfg::GW_REG ? T::P * C : Cfg::WAVES * T::P * kWave * Cfg::CPL;
  __shared__ float wl[Cfg::WL_LDS ? T::P * C : 1];
  __shared__ float gws[GWS];
  __shared__ float xch[Cfg::WAVES][kWave * NI];
  __shared__ int xsrc[Cfg::WAVES][Cfg::G];
  if constexpr (Cfg::WL_LDS)
    for (int i = threadIdx.x; i < T::P * C; i += Cfg::THREADS) wl[i] = w[(i / C) * CT + i % C];
  for (int i = threadIdx.x; i < GWS; i += Cfg::THREADS) gws[i] = 0.0f;
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int g = lane / Cfg::CL;
  const int cl = lane % Cfg::CL;
  const bool rows = mode != 0, by_src = mode == 2;
  float* const xw = xch[wv];
  // path weight of channel c (LDS copy or through the caches)
  auto wld = [&](int p, int c) -> float {
    if constexpr (Cfg::WL_LDS) return wl[p * C + c];
    else return w[p * CT + c];
  };
  // grad_w sums of this lane's channels over all its edges: registers, or the wave's slots
  // [P][CPL][64] (slot of path p, channel c = cl + j CL at (p CPL + j) 64 + lane)
  float gacc[Cfg::GW_REG ? Cfg::CPL : 1][Cfg::GW_REG ? T::P : 1];
  if constexpr (Cfg::GW_REG) {
#pragma unroll
    for (int j = 0; j < Cfg::CPL; ++j)
#pragma unroll
      for (int p = 0; p < T::P; ++p) gacc[j][p] = 0.0f;
  }
  float* const gslot = gws + (Cfg::GW_REG ? 0 : wv * T::P * kWave * Cfg::CPL + lane);

  for (long long task = (long long)blockIdx.x * Cfg::WAVES + wv; task < ntasks;
       task += (long long)gridDim.x * Cfg::WAVES) {
    int e_beg = 0, e_end = 0, row = 0;
    if (rows) {
      row = (int)task;
      if (E > 0) {
        e_beg = min(max(row_ptr[row], 0), E);
        e_end = min(max(row_ptr[row + 1], e_beg), E);
      }
      if (by_src && gx != nullptr) {  // the row's grad_x sums (lane-private slots)
#pragma unroll
        for (int i = 0; i < NI; ++i) xw[kWave * i + lane] = 0.0f;
        wave_lds_sync();
      }
    } else {
      e_beg = (int)(task * Cfg::EPW);
      e_end = (int)min((long long)E, task * Cfg::EPW + Cfg::EPW);
    }
#pragma clang loop unroll(disable)
    for (int e0 = e_beg; e0 < e_end; e0 += Cfg::G) {  // wave-uniform rounds of G edges
      const int e = e0 + g;
      const bool valid = e < e_end;
      const int ee = valid ? e : e0;  // e0 < e_end: a real edge for the idle slots
      const float vx = vec[3 * (size_t)ee], vy = vec[3 * (size_t)ee + 1], vz = vec[3 * (size_t)ee + 2];
      const int s = by_src ? row : clamp_index(src[ee], N);
      const int d = mode == 1 ? row : clamp_index(dst[ee], N);
      const So2Frame<L> f(vx, vy, vz);
      const float on = valid ? 1.0f : 0.0f;  // idle slots add nothing
      float gxe = 0.0f, gye = 0.0f;
      static_for<0, Cfg::CPL>([&](auto jj) {
        constexpr int j = decltype(jj)::value;
        if constexpr (j > 0) __builtin_amdgcn_sched_barrier(0);  // one channel at a time
        const int c = cl + j * Cfg::CL;
        float xr[K], gr[K];
        load_vec<K>(x + ((size_t)s * CT + c) * K, xr);
        load_vec<K>(gout + ((size_t)d * CT + c) * K, gr);
        so2_rotate_in<L, K>(xr, f);
        so2_rotate_in<L, K>(gr, f);
        // two walks of the sparse coupling (by path, then output component), so that at most three
        // K-vectors are live: A: t = (P_p x')[mu3], u'[mu3] += w_p t, grad_w[p] += g'[mu3] t;
        // B: v'[mu1] += w_p c g'[mu3]
        {
          float u[K];
#pragma unroll
          for (int k = 0; k < K; ++k) u[k] = 0.0f;
          // each path's weight is read from LDS one path ahead; the scheduling barriers at the path
          // boundaries keep the compiler from hoisting all P reads (P registers) to the top
          float wp = 0.0f, kp = 0.0f, t = 0.0f, tp = 0.0f, wn = wld(T::terms[0].p, c);
          static_for<0, T::NT>([&](auto ii) {
            constexpr int i = decltype(ii)::value;
            constexpr eqtp_gen::So2Term tm = T::terms[i];
            constexpr bool p_first = i == 0 || T::terms[i - 1].p != tm.p;
            constexpr bool p_last = i + 1 == T::NT || T::terms[i + 1].p != tm.p;
            constexpr bool run_first = p_first || T::terms[i - 1].mu3 != tm.mu3;
            constexpr bool run_last = p_last || T::terms[i + 1].mu3 != tm.mu3;
            if constexpr (p_first) {
              __builtin_amdgcn_sched_barrier(0);
              kp = tm.l2 > 0 ? f.keep * on : on;  // a zero vector drops the paths with l2 > 0
              wp = wn * kp;
              tp = 0.0f;
              constexpr int np = next_path_after<T>(i);
              if constexpr (np >= 0) wn = wld(np, c);
            }
            t = run_first ? tm.c * xr[tm.mu1] : fmaf(tm.c, xr[tm.mu1], t);
            if constexpr (run_last) {
              u[tm.mu3] = fmaf(wp, t, u[tm.mu3]);
              // the empty asm keeps each update where it is: sunk to their use after the walk, the
              // updates would hold every run's partial sum and weight live until then
              asm volatile("" : "+v"(u[tm.mu3]));
              tp = fmaf(gr[tm.mu3], t, tp);
            }
            if constexpr (p_last) {
              if constexpr (Cfg::GW_REG) gacc[j][tm.p] = fmaf(kp, tp, gacc[j][tm.p]);
              else gslot[(tm.p * Cfg::CPL + j) * kWave] = fmaf(kp, tp, gslot[(tm.p * Cfg::CPL + j) * kWave]);
            }
          });
          __builtin_amdgcn_sched_barrier(0);
          gxe -= gen_form<K, false>(u, gr);
          __builtin_amdgcn_sched_barrier(0);
          gye += gen_form<K, true>(u, gr);
        }
        __builtin_amdgcn_sched_barrier(0);  // walk B's loads stay after walk A (bounded live range)
        float v[K];
#pragma unroll
        for (int k = 0; k < K; ++k) v[k] = 0.0f;
        {
          int co = c;  // opaque: walk B reloads the weights instead of keeping walk A's P values live
          asm volatile("" : "+v"(co));
          float wp = 0.0f, qg = 0.0f, wn = wld(T::terms[0].p, co);
          static_for<0, T::NT>([&](auto ii) {
            constexpr int i = decltype(ii)::value;
            constexpr eqtp_gen::So2Term tm = T::terms[i];
            constexpr bool p_first = i == 0 || T::terms[i - 1].p != tm.p;
            constexpr bool run_first = p_first || T::terms[i - 1].mu3 != tm.mu3;
            if constexpr (p_first) {
              __builtin_amdgcn_sched_barrier(0);
              wp = wn * (tm.l2 > 0 ? f.keep * on : on);
              constexpr int np = next_path_after<T>(i);
              if constexpr (np >= 0) wn = wld(np, co);
            }
            if constexpr (run_first) qg = wp * gr[tm.mu3];
            v[tm.mu1] = fmaf(tm.c, qg, v[tm.mu1]);
            asm volatile("" : "+v"(v[tm.mu1]));
          });
        }
        __builtin_amdgcn_sched_barrier(0);
        gxe -= gen_form<K, false>(v, xr);
        __builtin_amdgcn_sched_barrier(0);
        gye += gen_form<K, true>(v, xr);
        __builtin_amdgcn_sched_barrier(0);
        if (gx != nullptr) {
          so2_rotate_out<L, K>(v, f);
          float* const xs = xw + (g * C + c) * K;
          if (by_src) {
#pragma unroll
            for (int k = 0; k < K; ++k) xs[k] += v[k];
          } else {
#pragma unroll
            for (int k = 0; k < K; ++k) xs[k] = v[k];
          }
        }
      });
      if (gvec != nullptr) {
#pragma unroll
        for (int off = 1; off < Cfg::CL; off <<= 1) {
          gxe += __shfl_xor(gxe, off);
          gye += __shfl_xor(gye, off);
        }
        if (valid && cl == 0) {  // zero for a zero vector
          const float r2 = vx * vx + vy * vy + vz * vz;
          float g0, g1, g2;
          frame_gradient<L>(f, gxe, gye, r2 > 0.0f ? rsqrtf(r2) : 0.0f, g0, g1, g2);
          float* gv = gvec + 3 * (by_src ? (size_t)clamp_index(perm[e], E) : (size_t)e);
          if constexpr (GV_ADD) {
            gv[0] += g0;
            gv[1] += g1;
            gv[2] += g2;
          } else {
            gv[0] = g0;
            gv[1] = g1;
            gv[2] = g2;
          }
        }
      }
      if (gx != nullptr && !by_src) {
        if (cl == 0) xsrc[wv][g] = valid ? s : -1;
        wave_lds_sync();
        // the lane index passes through an empty asm statement so that the NI addresses below are
        // formed here, not hoisted out of the edge loop (NI more live registers for the whole kernel)
        int ln = lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int fi = kWave * i + ln;
          const int sr = xsrc[wv][fi / MSG];
          if (sr >= 0) unsafeAtomicAdd(gx + (size_t)sr * (CT * K) + fi % MSG, xw[fi]);
        }
        wave_lds_sync();
      }
    }
    if (by_src && gx != nullptr) {  // the edge groups' sums, one coalesced store of the row (zeros if no edges)
      wave_lds_sync();
      int ln = lane;
      asm volatile("" : "+v"(ln));
      for (int f = ln; f < MSG; f += kWave) {
        float t = 0.0f;
#pragma unroll
        for (int gg = 0; gg < Cfg::G; ++gg) t += xw[gg * MSG + f];
        gx[(size_t)row * (CT * K) + f] = t;
      }
      wave_lds_sync();
    }
  }
  if (gw != nullptr) {
    if constexpr (Cfg::GW_REG) {
#pragma unroll
      for (int j = 0; j < Cfg::CPL; ++j)
#pragma unroll
        for (int p = 0; p < T::P; ++p) atomicAdd(&gws[p * C + cl + j * Cfg::CL], gacc[j][p]);
      __syncthreads();
      for (int i = threadIdx.x; i < T::P * C; i += Cfg::THREADS) unsafeAtomicAdd(gw + (i / C) * CT + i % C, gws[i]);
    } else {
      __syncthreads();
      for (int i = threadIdx.x; i < T::P * C; i += Cfg::THREADS) {
        const int p = i / C, c = i % C, j = c / Cfg::CL, cc = c % Cfg::CL;
        float sum = 0.0f;
        for (int ww = 0; ww < Cfg::WAVES; ++ww)
          for (int gg = 0; gg < Cfg::G; ++gg)
            sum += gws[ww * T::P * kWave * Cfg::CPL + (p * Cfg::CPL + j) * kWave + gg * Cfg::CL + cc];
        unsafeAtomicAdd(gw + p * CT + c, sum);
      }
    }
  }
}

// c0: the first channel this launch covers (rows CT channels wide; the zero fills cover every half and run
// with the first)
template <int L, int PS, int C, int CT = C>
static hipError_t launch_bwd_so2_t(const BwdArgs& a, int c0 = 0) {
  using Cfg = So2BwdCfg<L, PS, C>;
  using T = So2Tables<L, PS>;
  constexpr int K = num_comp(L);
  hipError_t err;
  if (c0 == 0) {
    // grouped by source every row's grad_x is written once (zeros without edges); else a sum of atomics
    if (a.gx && !a.by_src && (err = launch_fill_zero(a.gx, a.N * CT * K, a.stream)) != hipSuccess) return err;
    if (a.gw && (err = launch_fill_zero(a.gw, (int64_t)T::P * CT, a.stream)) != hipSuccess) return err;
  }
  const int mode = a.by_src ? 2 : a.row_ptr != nullptr ? 1 : 0;
  const long long ntasks = mode != 0 ? a.N : (a.E + Cfg::EPW - 1) / Cfg::EPW;
  if (ntasks == 0 || (a.E == 0 && !(a.by_src && a.gx))) return hipGetLastError();
  const int64_t want = (int64_t)num_cus() * Cfg::PER_CU;
  const int64_t need = (ntasks + Cfg::WAVES - 1) / Cfg::WAVES;
  const size_t ko = (size_t)c0 * K;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)(need < want ? need : want)), dim3(Cfg::THREADS), 0, a.stream,
                       (int)a.N, (int)a.E, ntasks, mode, a.row_ptr, a.vec, a.src, a.dst, a.perm,
                       a.x ? a.x + ko : nullptr, a.w + c0, a.gout + ko, a.gx ? a.gx + ko : nullptr,
                       a.gw ? a.gw + c0 : nullptr, a.gvec);
  };
  if (c0 == 0) go(conv_bwd_so2_kernel<L, PS, C, CT, false>);
  else go(conv_bwd_so2_kernel<L, PS, C, CT, true>);
  return hipGetLastError();
}

template <int L, int PS>
static hipError_t dispatch_bwd_so2_c(const BwdArgs& a) {
  switch (a.C) {
    case 8: return launch_bwd_so2_t<L, PS, 8>(a);
    case 16: return launch_bwd_so2_t<L, PS, 16>(a);
    case 32: return launch_bwd_so2_t<L, PS, 32>(a);
    case 64: return launch_bwd_so2_t<L, PS, 64>(a);
    case 128:
      if constexpr (L <= 2) {
        return launch_bwd_so2_t<L, PS, 128>(a);
      } else {  // two 64-channel halves: two channels per lane do not fit the registers above lmax 4, and from
                // lmax 3 they hold one wave per SIMD where the halves keep two
        const hipError_t err = launch_bwd_so2_t<L, PS, 64, 128>(a, 0);
        return err != hipSuccess ? err : launch_bwd_so2_t<L, PS, 64, 128>(a, 64);
      }
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_conv_backward_so2(const BwdArgs& a) {
  switch (a.lmax * 2 + a.path_set) {
    case 0: return dispatch_bwd_so2_c<0, 0>(a);
    case 1: return dispatch_bwd_so2_c<0, 1>(a);
    case 2: return dispatch_bwd_so2_c<1, 0>(a);
    case 3: return dispatch_bwd_so2_c<1, 1>(a);
    case 4: return dispatch_bwd_so2_c<2, 0>(a);
    case 5: return dispatch_bwd_so2_c<2, 1>(a);
    case 6: return dispatch_bwd_so2_c<3, 0>(a);
    case 7: return dispatch_bwd_so2_c<3, 1>(a);
    case 8: return dispatch_bwd_so2_c<4, 0>(a);
    case 9: return dispatch_bwd_so2_c<4, 1>(a);
    case 10: return dispatch_bwd_so2_c<5, 0>(a);
    case 11: return dispatch_bwd_so2_c<5, 1>(a);
    case 12: return dispatch_bwd_so2_c<6, 0>(a);
    case 13: return dispatch_bwd_so2_c<6, 1>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace eqtp
