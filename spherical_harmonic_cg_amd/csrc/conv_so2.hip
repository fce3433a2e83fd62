// conv_so2.hip -- the fused convolution in the edge-aligned (SO(2)) form, for
// lmax up to 6 (E2Former-V2 page, section 2.1 "derivation of EAAS").
//
// It computes what the Clebsch-Gordan form computes (Batmobile page, sections
// "2. register intermediate computation" and "3. operator fusion"):
//   out[n,c,mu3] = sum_{e: dst_e = n} sum_p w[p,c] sum_{mu1,mu2} C^p[mu1,mu2,mu3] x[src_e,c,mu1] Y_mu2(vec_e),
// by the equivariance of the coupling: with a rotation R_e that takes the
// edge direction to the z axis and D(R) its action on the real harmonics
// (Y(R u) = D(R) Y(u)),
//   message_e = D(R_e)^T  P(D(R_e) x[src_e]),
// where P is the coupling with the harmonics of the z axis, which are zero
// except for m = 0: each output component receives only input components of
// the same |m| (the page's sparse re-indexing; 624 terms instead of 6460 at
// lmax 6).  R_e = R_y(-theta) R_z(-phi) for the direction (theta, phi), and
// D(R_y(b)) = J^T D(R_z(b)) J with the constant J = D(R_x(pi/2)), so
//   D(R_e)   = J^T Z(-theta) J Z(-phi),   D(R_e)^T = Z(phi) J^T Z(theta) J,
// where Z(a) rotates every (m cos, m sin) component pair by m a.  No harmonic
// is evaluated and no per-edge matrix is built: the rotations are two
// sparse constant matrices (J, J^T: 119 entries up to lmax 6, immediates)
// and four pair rotations per edge and channel.  Tables and their checks:
// gen_so2_table.py.
//
// A zero edge vector: harmonics of degree > 0 are zero there, so the paths
// with l2 > 0 are dropped for that edge and the rotation is the identity.
//
// Lane mapping as in conv_edge.hip: lane = channel (C <= 64: 64/C edges per
// wave; C = 128: two channels per lane).  dst-sorted edges: one wave per
// destination row, lane groups combined with xor shuffles (deterministic);
// unsorted edges: contiguous edge runs per wave, messages added with fp32
// atomics after an LDS exchange (256 contiguous bytes per instruction).
// The path weights are staged once per workgroup in LDS ([P][C]).
#include <type_traits>

#include "eqtp_device.hpp"
#include "eqtp_kernels.hpp"
#include "so2_device.hpp"

namespace eqtp {

template <int C>
struct So2Cfg {
  static constexpr int CPL = C > 64 ? C / 64 : 1;  // channels per lane
  static constexpr int CL = C / CPL;               // lanes per edge group
  static constexpr int G = kWave / CL;             // edge groups per wave
  static constexpr int WAVES = 4;
  static constexpr int THREADS = WAVES * kWave;
  static constexpr int EPW = 8 * G;                // edges per wave, unsorted mode
};

// acc += D(R_e)^T P_w(D(R_e) v) for one channel (the radial kernel below; the
// fixed-weight kernels keep the same steps inline in So2Msg): v (the source features, K
// components) is rotated into the edge frame in place, coupled through the
// sparse table with path weight wfn(p) (dropped for l2 > 0 when the vector is
// zero), and the result rotated back and added into acc.
template <int L, int PS, int K, class WFn>
__device__ __forceinline__ void so2_message(float (&v)[K], const So2Frame<L>& f, WFn&& wfn, float (&acc)[K]) {
  using T = So2Tables<L, PS>;
  // into the edge frame: J^T Z(-theta) J Z(-phi)
  apply_z<L>(v, f.cp, f.sp, -1.0f);
  apply_j<K, false>(v);
  apply_z<L>(v, f.ct, f.st, -1.0f);
  apply_j<K, true>(v);
  // sparse coupling, one weight per path, one run per (path, output)
  float m[K];
#pragma unroll
  for (int k = 0; k < K; ++k) m[k] = 0.0f;
  float wp = 0.0f, t = 0.0f;
  static_for<0, T::NT>([&](auto ii) {
    constexpr int i = decltype(ii)::value;
    constexpr eqtp_gen::So2Term tm = T::terms[i];
    constexpr bool p_first = i == 0 || T::terms[i - 1].p != tm.p;
    constexpr bool run_first = p_first || T::terms[i - 1].mu3 != tm.mu3;
    constexpr bool run_last = i + 1 == T::NT || T::terms[i + 1].p != tm.p || T::terms[i + 1].mu3 != tm.mu3;
    if constexpr (p_first) {
      wp = wfn(std::integral_constant<int, tm.p>{});
      if constexpr (tm.l2 > 0) wp *= f.keep;
    }
    t = run_first ? tm.c * v[tm.mu1] : fmaf(tm.c, v[tm.mu1], t);
    if constexpr (run_last) m[tm.mu3] = fmaf(wp, t, m[tm.mu3]);
  });
  // back to the global frame: Z(phi) J^T Z(theta) J, added into acc
  apply_j<K, false>(m);
  apply_z<L>(m, f.ct, f.st, 1.0f);
  apply_j<K, true>(m);
  apply_z<L>(m, f.cp, f.sp, 1.0f);
#pragma unroll
  for (int k = 0; k < K; ++k) acc[k] += m[k];
}

// K consecutive features from xp (16-byte aligned when K % 4 == 0)
template <int K>
__device__ __forceinline__ void load_feat(const float* __restrict__ xp, float (&v)[K]) {
  if constexpr (K % 4 == 0) {
#pragma unroll
    for (int q = 0; q < K / 4; ++q) {
      const f4 t4 = reinterpret_cast<const f4*>(xp)[q];
      v[4 * q] = t4[0];
      v[4 * q + 1] = t4[1];
      v[4 * q + 2] = t4[2];
      v[4 * q + 3] = t4[3];
    }
  } else {
#pragma unroll
    for (int k = 0; k < K; ++k) v[k] = xp[k];
  }
}

// CT: channels per node row of x (C, or 128 when a C = 128 problem runs as two
// 64-channel halves, x and w then pointing at the half's first channel)
template <int L, int PS, int C, int CT = C>
struct So2Msg {
  using T = So2Tables<L, PS>;
  using Cfg = So2Cfg<C>;
  static constexpr int K = num_comp(L);

  // acc[j][:] += message of edge e for channels cl + j*CL; wl = weights [P][C] in LDS
  __device__ __forceinline__ static void run(int e, int N, int cl, const float* __restrict__ vec,
                                             const int* __restrict__ src, const float* __restrict__ x,
                                             const float* wl, float (&acc)[Cfg::CPL][K]) {
    const float vx = vec[3 * (size_t)e], vy = vec[3 * (size_t)e + 1], vz = vec[3 * (size_t)e + 2];
    const int s = clamp_index(src[e], N);
    // edge frame: cos/sin of phi and theta (identity for a zero vector or
    // along the z axis, where phi is free)
    const float r2 = vx * vx + vy * vy + vz * vz;
    const bool nz = r2 > 0.0f;
    const float inv_r = nz ? rsqrtf(r2) : 0.0f;
    const float ux = vx * inv_r, uy = vy * inv_r, uz = nz ? vz * inv_r : 1.0f;
    const float rho2 = ux * ux + uy * uy;
    const bool tilt = rho2 > 0.0f;
    const float inv_rho = tilt ? rsqrtf(rho2) : 0.0f;
    float cp[L + 1], sp[L + 1], ct[L + 1], st[L + 1];
    angle_powers<L>(tilt ? ux * inv_rho : 1.0f, tilt ? uy * inv_rho : 0.0f, cp, sp);
    angle_powers<L>(uz, tilt ? rho2 * inv_rho : 0.0f, ct, st);
    const float keep = nz ? 1.0f : 0.0f;  // paths with l2 > 0 vanish for a zero vector

#pragma unroll
    for (int j = 0; j < Cfg::CPL; ++j) {
      float v[K];
      const float* xp = x + ((size_t)s * CT + cl + j * Cfg::CL) * K;
      if constexpr (K % 4 == 0) {
#pragma unroll
        for (int q = 0; q < K / 4; ++q) {
          const f4 t4 = reinterpret_cast<const f4*>(xp)[q];
          v[4 * q] = t4[0];
          v[4 * q + 1] = t4[1];
          v[4 * q + 2] = t4[2];
          v[4 * q + 3] = t4[3];
        }
      } else {
#pragma unroll
        for (int k = 0; k < K; ++k) v[k] = xp[k];
      }
      // into the edge frame: J^T Z(-theta) J Z(-phi)
      apply_z<L>(v, cp, sp, -1.0f);
      apply_j<K, false>(v);
      apply_z<L>(v, ct, st, -1.0f);
      apply_j<K, true>(v);
      // sparse coupling, one weight per path, one run per (path, output)
      float m[K];
#pragma unroll
      for (int k = 0; k < K; ++k) m[k] = 0.0f;
      float wp = 0.0f, t = 0.0f;
      static_for<0, T::NT>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
        constexpr eqtp_gen::So2Term tm = T::terms[i];
        constexpr bool p_first = i == 0 || T::terms[i - 1].p != tm.p;
        constexpr bool run_first = p_first || T::terms[i - 1].mu3 != tm.mu3;
        constexpr bool run_last = i + 1 == T::NT || T::terms[i + 1].p != tm.p || T::terms[i + 1].mu3 != tm.mu3;
        if constexpr (p_first) {
          wp = wl[tm.p * C + cl + j * Cfg::CL];
          if constexpr (tm.l2 > 0) wp *= keep;
        }
        t = run_first ? tm.c * v[tm.mu1] : fmaf(tm.c, v[tm.mu1], t);
        if constexpr (run_last) m[tm.mu3] = fmaf(wp, t, m[tm.mu3]);
      });
      // back to the global frame: Z(phi) J^T Z(theta) J, added into acc
      apply_j<K, false>(m);
      apply_z<L>(m, ct, st, 1.0f);
      apply_j<K, true>(m);
      apply_z<L>(m, cp, sp, 1.0f);
#pragma unroll
      for (int k = 0; k < K; ++k) acc[j][k] += m[k];
    }
  }
};

template <int L, int PS, int C, bool ATOMIC, int CT = C>
__global__ __launch_bounds__(So2Cfg<C>::THREADS) void conv_so2_kernel(int N, int E, const int* __restrict__ row_ptr,
                                                                      const float* __restrict__ vec,
                                                                      const int* __restrict__ src,
                                                                      const int* __restrict__ dst,
                                                                      const float* __restrict__ x,
                                                                      const float* __restrict__ w,
                                                                      float* __restrict__ out) {
  using Cfg = So2Cfg<C>;
  using T = So2Tables<L, PS>;
  using M = So2Msg<L, PS, C, CT>;
  constexpr int K = num_comp(L);
  __shared__ float wl[T::P * C];
  for (int i = threadIdx.x; i < T::P * C; i += Cfg::THREADS) wl[i] = w[(i / C) * CT + i % C];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int g = lane / Cfg::CL;
  const int cl = lane % Cfg::CL;

  constexpr int MSG = C * K;        // floats per edge message (of this kernel's channels)
  constexpr int NI = Cfg::CPL * K;  // floats per lane of one round's messages
  // sorted rows at lmax >= 4 sum the messages in LDS (the lane's own slots)
  // rather than in registers, which the rotations and the coupling need
  constexpr bool LDS_ACC = !ATOMIC && K > 16;
  constexpr bool XCH = ATOMIC || LDS_ACC;
  __shared__ float xch[XCH ? Cfg::WAVES : 1][XCH ? kWave * NI : 1];
  float acc[Cfg::CPL][K];
  if constexpr (!ATOMIC) {
    const int row = blockIdx.x * Cfg::WAVES + wv;
    if (row >= N) return;
    int e_beg = 0, e_end = 0;
    if (E > 0) {
      e_beg = min(max(row_ptr[row], 0), E);
      e_end = min(max(row_ptr[row + 1], e_beg), E);
    }
    if constexpr (LDS_ACC) {
      float* const xw = xch[wv];
#pragma unroll
      for (int i = 0; i < NI; ++i) xw[kWave * i + lane] = 0.0f;
      wave_lds_sync();
#pragma clang loop unroll(disable)
      for (int e0 = e_beg; e0 < e_end; e0 += Cfg::G) {  // wave-uniform rounds of G edges
        const int e = e0 + g;
#pragma unroll
        for (int j = 0; j < Cfg::CPL; ++j)
#pragma unroll
          for (int k = 0; k < K; ++k) acc[j][k] = 0.0f;
        if (e < e_end) M::run(e, N, cl, vec, src, x, wl, acc);
        __builtin_amdgcn_sched_barrier(0);  // keep the LDS sums after the message (bounded live range)
#pragma unroll
        for (int j = 0; j < Cfg::CPL; ++j)
#pragma unroll
          for (int k = 0; k < K; ++k) xw[(g * C + cl + j * Cfg::CL) * K + k] += acc[j][k];
        wave_lds_sync();
      }
      wave_lds_sync();
#pragma unroll
      for (int j = 0; j < Cfg::CPL; ++j)
#pragma unroll
        for (int k = 0; k < K; ++k) {
          float t = 0.0f;
#pragma unroll
          for (int gg = 0; gg < Cfg::G; ++gg) t += xw[(gg * C + cl + j * Cfg::CL) * K + k];
          acc[j][k] = t;
        }
    } else {
#pragma unroll
      for (int j = 0; j < Cfg::CPL; ++j)
#pragma unroll
        for (int k = 0; k < K; ++k) acc[j][k] = 0.0f;
      for (int e = e_beg + g; e < e_end; e += Cfg::G) M::run(e, N, cl, vec, src, x, wl, acc);
#pragma unroll
      for (int off = Cfg::CL; off < kWave; off <<= 1)
#pragma unroll
        for (int j = 0; j < Cfg::CPL; ++j)
#pragma unroll
          for (int k = 0; k < K; ++k) acc[j][k] += __shfl_xor(acc[j][k], off);
    }
    if (g == 0) {
#pragma unroll
      for (int j = 0; j < Cfg::CPL; ++j) {
        float* op = out + ((size_t)row * CT + cl + j * Cfg::CL) * K;
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
      if (valid) M::run(e, N, cl, vec, src, x, wl, acc);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < Cfg::CPL; ++j)
#pragma unroll
        for (int k = 0; k < K; ++k) xw[(g * C + cl + j * Cfg::CL) * K + k] = acc[j][k];
      if (cl == 0) xdst[wv][g] = valid ? clamp_index(dst[e], N) : -1;
      wave_lds_sync();
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int f = kWave * i + lane;
        const int d = xdst[wv][f / MSG];
        if (d >= 0) unsafeAtomicAdd(out + (size_t)d * (CT * K) + f % MSG, xw[f]);
      }
      wave_lds_sync();
    }
  }
}

// Per-edge messages in the edge-aligned form (the page's fused-kernel output
// [E, C, K], no destination sum): the wave's store of one edge covers its
// C*K*4 contiguous bytes.
template <int L, int PS, int C, int CT = C>
__global__ __launch_bounds__(So2Cfg<C>::THREADS) void conv_so2_msg_kernel(int N, int E, const float* __restrict__ vec,
                                                                          const int* __restrict__ src,
                                                                          const float* __restrict__ x,
                                                                          const float* __restrict__ w,
                                                                          float* __restrict__ msg) {
  using Cfg = So2Cfg<C>;
  using T = So2Tables<L, PS>;
  using M = So2Msg<L, PS, C, CT>;
  constexpr int K = num_comp(L);
  __shared__ float wl[T::P * C];
  for (int i = threadIdx.x; i < T::P * C; i += Cfg::THREADS) wl[i] = w[(i / C) * CT + i % C];
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int g = lane / Cfg::CL;
  const int cl = lane % Cfg::CL;
  const long long base = ((long long)blockIdx.x * Cfg::WAVES + wv) * Cfg::EPW;
  const int e_end = (int)min((long long)E, base + Cfg::EPW);
#pragma clang loop unroll(disable)
  for (int e = (int)base + g; e < e_end; e += Cfg::G) {
    float acc[Cfg::CPL][K];
#pragma unroll
    for (int j = 0; j < Cfg::CPL; ++j)
#pragma unroll
      for (int k = 0; k < K; ++k) acc[j][k] = 0.0f;
    M::run(e, N, cl, vec, src, x, wl, acc);
#pragma unroll
    for (int j = 0; j < Cfg::CPL; ++j) {
      float* op = msg + ((size_t)e * CT + cl + j * Cfg::CL) * K;
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

// ---------------------------------------------------------------------------
// Radial weights, dst-sorted edges, lmax <= 3, C a multiple of 16.
// The path weights of an edge are w_e[p,c] = sum_b R_b(|vec_e|) W[b, p*C + c]
// with the 8 radial functions R_b (eqtp_device.hpp).  For a batch of 16 edges
// of one row and a block of 16 channels that is a [16 x 8] x [8 x 16] product
// per path: two v_mfma_f32_16x16x4_f32 with A = R (rows = edges, shared by all
// paths) and B = W (the workgroup's LDS copy of the block's columns), so W is
// read once per 16 edges instead of once per edge.  A's rows are the batch's
// edges in the order k + 4i of row 4k + i, so the MFMA leaves w of
// (edge k + 4i, channel j) in lane (j, k), which is how the rest of the batch
// runs: lane (j, k) takes the batch's edges k, k+4, k+8, k+12 for channel j
// through the edge-aligned coupling (rotate in, sparse coupling with w,
// rotate back) and sums the messages in registers.  A row's last, partial
// batch of n edges then stops after ceil(n/4) of the 4 slots.  The four edge
// groups of a lane's channel are combined with xor shuffles after the row
// (deterministic).  Each edge's frame (cos/sin of m phi, m theta) and source
// index are computed once per batch, from the edge vector the lane loads for
// its A row, and shared through the wave's LDS.
// Work unit: one wave per (row, 16-channel block); a workgroup's 4 waves take
// 4 consecutive rows of one block; workgroups are numbered block-major.  The
// parity path set fits 168 VGPRs (3 waves per SIMD); the SO(3) set keeps 2.
// ---------------------------------------------------------------------------
constexpr int kSo2RadialBasis = 8;
// Per-edge basis of width 64 (the hidden layer of a radial network, given by
// the caller in memory): w_e[p,c] = sum_k phi_e[k] W[k, p*C + c] is the same
// product with K = 64, 16 MFMAs per path.  phi is stored per edge as [4][16]:
// hidden unit k = 4 i + q sits at q * 16 + i, so lane group q reads its 16
// A values of an edge as 4 contiguous 16-byte loads.  The workgroup holds the
// block's 64 x P x 16 slice of W (94 KB at P = 23) and runs 8 waves, two per
// SIMD, on it.
constexpr int kSo2BasisWidth = 64;

template <int NB>
struct So2RadialCfg {
  static constexpr int WAVES = NB == kSo2RadialBasis ? 4 : 8;
};

template <int L, int PS, int C, int NB>
__global__ __launch_bounds__(So2RadialCfg<NB>::WAVES * 64) __attribute__((amdgpu_waves_per_eu(
    NB == kSo2RadialBasis ? (PS == 0 ? 3 : 2) : (PS == 0 ? 2 : 1)))) void conv_so2_radial_kernel(
    int N, int E, const int* __restrict__ row_ptr, const float* __restrict__ vec, const int* __restrict__ src,
    const float* __restrict__ x, const float* __restrict__ w, float* __restrict__ out, float inv_rc,
    const float* __restrict__ phi) {
  using T = So2Tables<L, PS>;
  constexpr int K = num_comp(L);
  constexpr int P = T::P;
  constexpr int NBLK = C / 16;
  constexpr int WAVES = So2RadialCfg<NB>::WAVES;
  constexpr bool BASIS = NB != kSo2RadialBasis;
  static_assert(C % 16 == 0 && L <= 3, "radial edge-aligned kernel: C multiple of 16, lmax <= 3");
  static_assert(NB == kSo2RadialBasis || NB == kSo2BasisWidth, "basis width 8 (radial functions) or 64");
  using Frame = So2Frame<L>;
  __shared__ float wl[NB * P * 16];  // [b][p][channel of the block]
  // the current batch's 16 edge frames and sources, per wave (computed once per batch, read by every
  // channel lane)
  __shared__ __attribute__((aligned(16))) float frm[WAVES][16 * Frame::FS];
  // block-major order: the workgroups in flight at any time share one channel
  // block, so the gathered slice of x (N * 16 * K floats) is what the caches
  // must hold, not all of x
  const int ngrp = (N + WAVES - 1) / WAVES;
  const int cb = (int)(blockIdx.x / ngrp) * 16;
  for (int i = threadIdx.x; i < NB * P * 16; i += WAVES * 64) {
    const int bp = i >> 4;  // b * P + p
    wl[i] = w[(size_t)bp * C + cb + (i & 15)];
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int row = (int)(blockIdx.x % ngrp) * WAVES + (threadIdx.x >> 6);
  if (row >= N) return;
  const int j = lane & 15;   // channel cb + j; A row (edge e0 + j) for the radial product
  const int kq = lane >> 4;  // edge group: edges kq + 4 i of each batch; A/B k index
  int e_beg = 0, e_end = 0;
  if (E > 0) {
    e_beg = min(max(row_ptr[row], 0), E);
    e_end = min(max(row_ptr[row + 1], e_beg), E);
  }
  float acc[K];
#pragma unroll
  for (int k = 0; k < K; ++k) acc[k] = 0.0f;
  for (int e0 = e_beg; e0 < e_end; e0 += 16) {
    // A operand of lane (j, kq): basis functions kq, 4 + kq, ... of the edge of A row j,
    // e0 + (j >> 2) + 4 (j & 3) (zeros past the row), and the frame and source of that edge, written by
    // the lanes of group 0 to the wave's LDS
    float av[NB / 4];
#pragma unroll
    for (int i = 0; i < NB / 4; ++i) av[i] = 0.0f;
    const int ar = (j >> 2) | ((j & 3) << 2);
    const int ea = e0 + ar;
    float ax = 0.0f, ay = 0.0f, az = 0.0f;
    int sa = 0;
    if (ea < e_end) {
      ax = vec[3 * (size_t)ea];
      ay = vec[3 * (size_t)ea + 1];
      az = vec[3 * (size_t)ea + 2];
      sa = clamp_index(src[ea], N);
      if constexpr (BASIS) {
        const f4* pr = reinterpret_cast<const f4*>(phi + (size_t)ea * NB + kq * (NB / 4));
#pragma unroll
        for (int q = 0; q < NB / 16; ++q) {
          const f4 v4 = pr[q];
#pragma unroll
          for (int r = 0; r < 4; ++r) av[4 * q + r] = v4[r];
        }
      } else {
        float R[NB];
        radial_basis<NB>(sqrtf(ax * ax + ay * ay + az * az), inv_rc, R);
        av[0] = kq == 0 ? R[0] : (kq == 1 ? R[1] : (kq == 2 ? R[2] : R[3]));
        av[1] = kq == 0 ? R[4] : (kq == 1 ? R[5] : (kq == 2 ? R[6] : R[7]));
      }
    }
    float* const wf = frm[threadIdx.x >> 6];
    wave_lds_sync();  // the previous batch's frames have been read
    if (kq == 0) {
      Frame(ax, ay, az).store(wf + ar * Frame::FS);
      reinterpret_cast<int*>(wf + ar * Frame::FS)[Frame::SRC] = sa;  // the edge's source, beside its frame
    }
    wave_lds_sync();
    // w of edges e0 + kq + 4 i, channel cb + j: wp[p][i]
    f4 wp[P];
    // basis functions 0..3 for every path first, then the next four accumulated (no back-to-back dependent
    // products)
#pragma unroll
    for (int p = 0; p < P; ++p)
      wp[p] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[0], wl[(kq * P + p) * 16 + j], f4{0.f, 0.f, 0.f, 0.f}, 0, 0,
                                                   0);
#pragma unroll
    for (int i = 1; i < NB / 4; ++i)
#pragma unroll
      for (int p = 0; p < P; ++p)
        wp[p] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i], wl[((4 * i + kq) * P + p) * 16 + j], wp[p], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (e0 + 4 * i >= e_end) break;  // no edge left for any lane (wave-uniform)
      const int e = e0 + kq + 4 * i;
      if (e < e_end) {
        Frame f;
        f.load(wf + (kq + 4 * i) * Frame::FS);
        const int s = reinterpret_cast<const int*>(wf + (kq + 4 * i) * Frame::FS)[Frame::SRC];
        float v[K];
        load_feat<K>(x + ((size_t)s * C + cb + j) * K, v);
        so2_message<L, PS>(v, f, [&](auto p) { return wp[decltype(p)::value][i]; }, acc);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < K; ++k) {
    acc[k] += __shfl_xor(acc[k], 16);
    acc[k] += __shfl_xor(acc[k], 32);
  }
  if (kq == 0) {
    float* op = out + ((size_t)row * C + cb + j) * K;
    if constexpr (K % 4 == 0) {
#pragma unroll
      for (int q = 0; q < K / 4; ++q)
        reinterpret_cast<f4*>(op)[q] = f4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
    } else {
#pragma unroll
      for (int k = 0; k < K; ++k) op[k] = acc[k];
    }
  }
}

template <int L, int PS, int C>
static hipError_t launch_so2_radial_t(const ConvArgs& a) {
  if (a.N == 0) return hipSuccess;
  if (a.phi != nullptr) {  // per-edge basis of width 64
    constexpr int WV = So2RadialCfg<kSo2BasisWidth>::WAVES;
    const long long blocks = (a.N + WV - 1) / WV * (C / 16);
    hipLaunchKernelGGL((conv_so2_radial_kernel<L, PS, C, kSo2BasisWidth>), dim3((unsigned)blocks), dim3(WV * 64), 0,
                       a.stream, (int)a.N, (int)a.E, a.row_ptr, a.vec, a.src, (const float*)a.x, a.w, a.out, 0.0f,
                       a.phi);
    return hipGetLastError();
  }
  constexpr int WV = So2RadialCfg<kSo2RadialBasis>::WAVES;
  const long long blocks = (a.N + WV - 1) / WV * (C / 16);
  hipLaunchKernelGGL((conv_so2_radial_kernel<L, PS, C, kSo2RadialBasis>), dim3((unsigned)blocks), dim3(WV * 64), 0,
                     a.stream, (int)a.N, (int)a.E, a.row_ptr, a.vec, a.src, (const float*)a.x, a.w, a.out,
                     1.0f / a.r_cut, nullptr);
  return hipGetLastError();
}

template <int L, int PS>
static hipError_t dispatch_so2_radial_c(const ConvArgs& a) {
  switch (a.C) {
    case 16: return launch_so2_radial_t<L, PS, 16>(a);
    case 32: return launch_so2_radial_t<L, PS, 32>(a);
    case 64: return launch_so2_radial_t<L, PS, 64>(a);
    case 128: return launch_so2_radial_t<L, PS, 128>(a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_conv_so2_radial(const ConvArgs& a) {
  switch (a.lmax * 2 + a.path_set) {
    case 0: return dispatch_so2_radial_c<0, 0>(a);
    case 1: return dispatch_so2_radial_c<0, 1>(a);
    case 2: return dispatch_so2_radial_c<1, 0>(a);
    case 3: return dispatch_so2_radial_c<1, 1>(a);
    case 4: return dispatch_so2_radial_c<2, 0>(a);
    case 5: return dispatch_so2_radial_c<2, 1>(a);
    case 6: return dispatch_so2_radial_c<3, 0>(a);
    case 7: return dispatch_so2_radial_c<3, 1>(a);
    default: return hipErrorInvalidValue;
  }
}

// c0: the first channel this launch covers (x, w and out offset by it; rows CT channels wide)
template <int L, int PS, int C, int CT = C>
static hipError_t launch_so2_t(const ConvArgs& a, int c0 = 0) {
  using Cfg = So2Cfg<C>;
  constexpr int K = num_comp(L);
  if (a.N == 0) return hipSuccess;
  const float* const x = (const float*)a.x + (size_t)c0 * K;
  const float* const w = a.w + c0;
  float* const out = a.out + (size_t)c0 * K;
  if (a.messages) {
    if (a.E == 0) return hipSuccess;
    const long long per_block = (long long)Cfg::WAVES * Cfg::EPW;
    const unsigned blocks = (unsigned)((a.E + per_block - 1) / per_block);
    hipLaunchKernelGGL((conv_so2_msg_kernel<L, PS, C, CT>), dim3(blocks), dim3(Cfg::THREADS), 0, a.stream, (int)a.N,
                       (int)a.E, a.vec, a.src, x, w, out);
    return hipGetLastError();
  }
  if (a.row_ptr != nullptr) {
    const unsigned blocks = (unsigned)((a.N + Cfg::WAVES - 1) / Cfg::WAVES);
    hipLaunchKernelGGL((conv_so2_kernel<L, PS, C, false, CT>), dim3(blocks), dim3(Cfg::THREADS), 0, a.stream,
                       (int)a.N, (int)a.E, a.row_ptr, a.vec, a.src, a.dst, x, w, out);
  } else {
    if (c0 == 0) {  // the whole output (every half) once
      hipError_t err = launch_fill_zero(a.out, a.N * CT * K, a.stream);
      if (err != hipSuccess) return err;
    }
    if (a.E == 0) return hipSuccess;
    const long long per_block = (long long)Cfg::WAVES * Cfg::EPW;
    const unsigned blocks = (unsigned)((a.E + per_block - 1) / per_block);
    hipLaunchKernelGGL((conv_so2_kernel<L, PS, C, true, CT>), dim3(blocks), dim3(Cfg::THREADS), 0, a.stream,
                       (int)a.N, (int)a.E, a.row_ptr, a.vec, a.src, a.dst, x, w, out);
  }
  return hipGetLastError();
}

template <int L, int PS>
static hipError_t dispatch_so2_c(const ConvArgs& a) {
  switch (a.C) {
    case 8: return launch_so2_t<L, PS, 8>(a);
    case 16: return launch_so2_t<L, PS, 16>(a);
    case 32: return launch_so2_t<L, PS, 32>(a);
    case 64: return launch_so2_t<L, PS, 64>(a);
    case 128:
      if constexpr (L <= 3) {
        return launch_so2_t<L, PS, 128>(a);
      } else {  // two 64-channel halves: two channels per lane do not fit the registers above lmax 4, and at
                // lmax 4 the halves are faster for dst-sorted edges and messages
        const hipError_t err = launch_so2_t<L, PS, 64, 128>(a, 0);
        return err != hipSuccess ? err : launch_so2_t<L, PS, 64, 128>(a, 64);
      }
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_conv_so2(const ConvArgs& a) {
  switch (a.lmax * 2 + a.path_set) {
    case 0: return dispatch_so2_c<0, 0>(a);
    case 1: return dispatch_so2_c<0, 1>(a);
    case 2: return dispatch_so2_c<1, 0>(a);
    case 3: return dispatch_so2_c<1, 1>(a);
    case 4: return dispatch_so2_c<2, 0>(a);
    case 5: return dispatch_so2_c<2, 1>(a);
    case 6: return dispatch_so2_c<3, 0>(a);
    case 7: return dispatch_so2_c<3, 1>(a);
    case 8: return dispatch_so2_c<4, 0>(a);
    case 9: return dispatch_so2_c<4, 1>(a);
    case 10: return dispatch_so2_c<5, 0>(a);
    case 11: return dispatch_so2_c<5, 1>(a);
    case 12: return dispatch_so2_c<6, 0>(a);
    case 13: return dispatch_so2_c<6, 1>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace eqtp
