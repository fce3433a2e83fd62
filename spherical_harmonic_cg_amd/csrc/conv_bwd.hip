// conv_bwd.hip -- gradients of the fused convolution with fixed path weights,
// evaluated edge by edge on the vector ALUs.
//
// Forward (Batmobile page, sections "2. register intermediate computation" and
// "3. operator fusion", with the destination sum):
//   out[n,c,mu3] = sum_{e: dst_e = n} sum_p w[p,c] sum_{mu1,mu2} C^p[mu1,mu2,mu3] x[src_e,c,mu1] Y_mu2(vec_e).
// For L = sum gout * out, per edge e = (s -> d) and channel c:
//   s1[p,mu1] = sum_{mu2,mu3} C^p Y[mu2] gout[d,c,mu3]
//     -> grad_x[s,c,mu1] += w[p,c] s1,   grad_w[p,c] += x[s,c,mu1] s1
//   s2[p,mu2] = sum_{mu1,mu3} C^p x[s,c,mu1] gout[d,c,mu3]
//     -> dL/dY_e[mu2] += w[p,c] s2 (summed over channels)
//   grad_vec[e] = sum_mu2 dL/dY_e[mu2] dY_mu2/dvec_e   (sh_grad_eval).
// The two sums walk the constexpr coupling table in (path, mu1) and (path,
// mu2) order so each partial sum is a contiguous run of immediates.
//
// Lane mapping as in the per-edge forward: lane = channel (C <= 64: 64/C edges
// per round, one per lane group; C = 128: two channels per lane).
//   * dst-sorted edges (row_ptr): one wavefront per destination row, so the
//     row's gout block is read once;
//   * unsorted edges (dst): each wave takes a contiguous run of edges.
// grad_x is a scatter into sources: a round's per-lane contributions are
// exchanged through LDS and added with fp32 atomics covering 256 contiguous
// bytes per instruction.  grad_w is accumulated in registers over all the
// wave's edges and added once per wave.  grad_vec is written per edge.
// The two walks are separate launches (PASS 1: grad_x and grad_w; PASS 2:
// grad_vec), so that each holds only its own accumulators: one launch doing
// both needs about 300 registers at lmax 3, which leaves one wave per SIMD.
#include "eqtp_device.hpp"
#include "eqtp_kernels.hpp"
#include "so2_device.hpp"

namespace eqtp {

// ---------------------------------------------------------------------------
// Gradient of the real harmonics with respect to the (unnormalised) edge
// vector: G[k][a] = dY_k / dvec_a.  Each Y_k of sh_eval is a polynomial p_k in the
// unit vector u = vec/|vec|; its gradient in u (written out per component
// below) is projected onto the sphere's tangent plane and divided by |vec|:
// G = (grad p - u (u . grad p)) / |vec|.  A zero vector gives G = 0 (Y is
// constant there).  Y is returned as by sh_eval.
// ---------------------------------------------------------------------------
template <int L>
__device__ __forceinline__ void sh_grad_eval(float vx, float vy, float vz, float (&Y)[16], float (&G)[16][3]) {
  using namespace eqtp_gen;
  sh_eval<L>(vx, vy, vz, Y);
  const float r2 = vx * vx + vy * vy + vz * vz;
  const bool nz = r2 > 0.0f;
  const float inv = nz ? rsqrtf(r2) : 0.0f;
  const float x = vx * inv, y = vy * inv, z = vz * inv;
  float g[16][3];
#pragma unroll
  for (int k = 0; k < 16; ++k) g[k][0] = g[k][1] = g[k][2] = 0.0f;
  if constexpr (L >= 1) {
    g[1][2] = kShC1;
    g[2][0] = -kShC1;
    g[3][1] = -kShC1;
  }
  if constexpr (L >= 2) {
    g[4][2] = 6.0f * kShC20 * z;
    g[5][0] = -kShC21 * z;
    g[5][2] = -kShC21 * x;
    g[6][1] = -kShC21 * z;
    g[6][2] = -kShC21 * y;
    g[7][0] = 2.0f * kShC22 * x;
    g[7][1] = -2.0f * kShC22 * y;
    g[8][0] = 2.0f * kShC22 * y;
    g[8][1] = 2.0f * kShC22 * x;
  }
  if constexpr (L >= 3) {
    const float zz = z * z, d = x * x - y * y;
    g[9][2] = kShC30 * (15.0f * zz - 3.0f);
    g[10][0] = -kShC31 * (5.0f * zz - 1.0f);
    g[10][2] = -10.0f * kShC31 * x * z;
    g[11][1] = -kShC31 * (5.0f * zz - 1.0f);
    g[11][2] = -10.0f * kShC31 * y * z;
    g[12][0] = 2.0f * kShC32 * x * z;
    g[12][1] = -2.0f * kShC32 * y * z;
    g[12][2] = kShC32 * d;
    g[13][0] = 2.0f * kShC32 * y * z;
    g[13][1] = 2.0f * kShC32 * x * z;
    g[13][2] = 2.0f * kShC32 * x * y;
    g[14][0] = -3.0f * kShC33 * d;
    g[14][1] = 6.0f * kShC33 * x * y;
    g[15][0] = -6.0f * kShC33 * x * y;
    g[15][1] = -3.0f * kShC33 * d;
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const float ug = x * g[k][0] + y * g[k][1] + z * g[k][2];
    G[k][0] = (g[k][0] - x * ug) * inv;
    G[k][1] = (g[k][1] - y * ug) * inv;
    G[k][2] = (g[k][2] - z * ug) * inv;
  }
}

// by_out positions ordered by a (path, component) key, stably: KEY 1 sorts by
// (p, mu1), KEY 2 by (p, mu2).  Runs of equal key are contiguous.
template <int L, int PS, int KEY>
struct TermOrder {
  using T = Tables<L, PS>;
  struct Idx {
    short v[T::NT > 0 ? T::NT : 1];
  };
  static constexpr int key(int i) { return T::by_out[i].p * 16 + (KEY == 1 ? T::by_out[i].mu1 : T::by_out[i].mu2); }
  static constexpr Idx make() {  // stable counting sort by key
    Idx a{};
    int pos[64 * 16 + 1] = {};
    for (int i = 0; i < T::NT; ++i) pos[key(i) + 1]++;
    for (int kk = 0; kk < 64 * 16; ++kk) pos[kk + 1] += pos[kk];
    for (int i = 0; i < T::NT; ++i) a.v[pos[key(i)]++] = (short)i;
    return a;
  }
  static constexpr Idx order = make();
  static constexpr const eqtp_gen::CgTerm& term(int j) { return T::by_out[order.v[j]]; }
  static constexpr bool first(int j) { return j == 0 || key(order.v[j - 1]) != key(order.v[j]); }
  static constexpr bool last(int j) { return j + 1 == T::NT || key(order.v[j + 1]) != key(order.v[j]); }
  // the terms of one path are contiguous too (the key is path-major)
  static constexpr int path(int j) { return T::by_out[order.v[j]].p; }
  static constexpr bool path_first(int j) { return j == 0 || path(j - 1) != path(j); }
  static constexpr bool path_last(int j) { return j + 1 == T::NT || path(j + 1) != path(j); }
};


template <int C>
struct BwdCfg {
  static constexpr int CPL = C > 64 ? C / 64 : 1;  // channels per lane
  static constexpr int CL = C / CPL;               // lanes per edge group
  static constexpr int G = kWave / CL;             // edge groups per wave
  static constexpr int WAVES = 4;
  static constexpr int THREADS = WAVES * kWave;
  static constexpr int EPW = 16 * G;               // edges per wave, unsorted mode
};

template <int L, int PS, int C, bool SORTED, int PASS>
__global__ __launch_bounds__(BwdCfg<C>::THREADS) void conv_bwd_kernel(
    int N, int E, const int* __restrict__ row_ptr, const float* __restrict__ vec, const int* __restrict__ src,
    const int* __restrict__ dst, const float* __restrict__ x, const float* __restrict__ w,
    const float* __restrict__ gout, float* __restrict__ gx, float* __restrict__ gw, float* __restrict__ gvec) {
  using Cfg = BwdCfg<C>;
  using T = Tables<L, PS>;
  using O1 = TermOrder<L, PS, 1>;
  using O2 = TermOrder<L, PS, 2>;
  constexpr int K = num_comp(L);
  constexpr int P = T::P;
  constexpr int MSG = C * K;         // floats per node block
  constexpr int NI = Cfg::CPL * K;   // atomic instructions per wave and round
  __shared__ float xch[Cfg::WAVES][kWave * NI];
  __shared__ int xsrc[Cfg::WAVES][Cfg::G];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int g = lane / Cfg::CL;
  const int cl = lane % Cfg::CL;
  float* const xw = xch[wv];

  if constexpr (PASS == 1) {
    if (gx == nullptr && gw == nullptr) return;
  } else {
    if (gvec == nullptr) return;
  }
  float wreg[Cfg::CPL][P];
  float gwacc[Cfg::CPL][PASS == 1 ? P : 1];
#pragma unroll
  for (int j = 0; j < Cfg::CPL; ++j) {
#pragma unroll
    for (int p = 0; p < P; ++p) wreg[j][p] = w[p * C + cl + j * Cfg::CL];
#pragma unroll
    for (int p = 0; p < (PASS == 1 ? P : 1); ++p) gwacc[j][p] = 0.0f;
  }

  float gv[Cfg::CPL][K];  // gout[d, channel, :]
  auto load_g = [&](int d) {
#pragma unroll
    for (int j = 0; j < Cfg::CPL; ++j)
#pragma unroll
      for (int k = 0; k < K; ++k) gv[j][k] = gout[((size_t)d * C + cl + j * Cfg::CL) * K + k];
  };

  // An edge's inputs, loaded one round ahead of their use.  Invalid slots
  // load an in-range edge (their results are discarded), so the loads carry
  // no branches.
  struct EdgeIn {
    float vx, vy, vz;
    int s;
    float xv[Cfg::CPL][K];
    float gd[SORTED ? 1 : Cfg::CPL][K];  // gout of the destination (unsorted edges)
  };
  auto fetch = [&](int e, bool valid, int e_alt) {
    EdgeIn in;
    const int ec = valid ? e : e_alt;
    in.vx = vec[3 * (size_t)ec];
    in.vy = vec[3 * (size_t)ec + 1];
    in.vz = vec[3 * (size_t)ec + 2];
    in.s = clamp_index(src[ec], N);
#pragma unroll
    for (int j = 0; j < Cfg::CPL; ++j)
#pragma unroll
      for (int k = 0; k < K; ++k) in.xv[j][k] = x[((size_t)in.s * C + cl + j * Cfg::CL) * K + k];
    if constexpr (!SORTED) {
      const int d = clamp_index(dst[ec], N);
#pragma unroll
      for (int j = 0; j < Cfg::CPL; ++j)
#pragma unroll
        for (int k = 0; k < K; ++k) in.gd[j][k] = gout[((size_t)d * C + cl + j * Cfg::CL) * K + k];
    }
    return in;
  };

  // one round: lane group g handles edge e (if valid) with inputs in.  The
  // (path, mu1) pass and the grad_x exchange finish before the (path, mu2)
  // pass starts, so their accumulators are never live together.
  auto round = [&](int e, bool valid, const EdgeIn& in) {
    float Y[16];
    if (valid) sh_eval<L>(in.vx, in.vy, in.vz, Y);
    if constexpr (PASS == 1) {
      float mx[Cfg::CPL][K];
#pragma unroll
      for (int j = 0; j < Cfg::CPL; ++j)
#pragma unroll
        for (int k = 0; k < K; ++k) mx[j][k] = 0.0f;
      if (valid) {
#pragma unroll
        for (int j = 0; j < Cfg::CPL; ++j) {
          const float(&gj)[K] = SORTED ? gv[j] : in.gd[SORTED ? 0 : j];
          // (path, mu1) runs: grad_x and grad_w
          float s1 = 0.0f;
          static_for<0, T::NT>([&](auto jj) {
            constexpr int q = decltype(jj)::value;
            constexpr eqtp_gen::CgTerm tm = O1::term(q);
            // (c * Y) * g per term: no product shared between terms, so no long-lived common subexpressions
            const float cy = tm.c * Y[tm.mu2];
            s1 = O1::first(q) ? cy * gj[tm.mu3] : fmaf(cy, gj[tm.mu3], s1);
            if constexpr (O1::last(q)) {
              mx[j][tm.mu1] = fmaf(wreg[j][tm.p], s1, mx[j][tm.mu1]);
              if constexpr (PASS == 1) gwacc[j][tm.p] = fmaf(in.xv[j][tm.mu1], s1, gwacc[j][tm.p]);
              __builtin_amdgcn_sched_barrier(0);  // keep runs apart: bounded live temporaries
            }
          });
        }
      }
      // grad_x: exchange the round's contributions so that atomic instruction
      // i adds floats 64i .. 64i+63 of the wave's G source blocks
      if (gx != nullptr) {
#pragma unroll
        for (int j = 0; j < Cfg::CPL; ++j)
#pragma unroll
          for (int k = 0; k < K; ++k) xw[(g * C + cl + j * Cfg::CL) * K + k] = mx[j][k];
        if (cl == 0) xsrc[wv][g] = valid ? in.s : -1;  // -1: no edge in this slot
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int f = kWave * i + lane;
          const int sd = xsrc[wv][f / MSG];
          if (sd >= 0) unsafeAtomicAdd(gx + (size_t)sd * MSG + f % MSG, xw[f]);
        }
        wave_lds_sync();
      }
    }
    if constexpr (PASS == 2) {
      float dy[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) dy[k] = 0.0f;
      if (valid) {
#pragma unroll
        for (int j = 0; j < Cfg::CPL; ++j) {
          const float(&gj)[K] = SORTED ? gv[j] : in.gd[SORTED ? 0 : j];
          // (path, mu2) runs: dL/dY
          float s2 = 0.0f;
          static_for<0, T::NT>([&](auto jj) {
            constexpr int q = decltype(jj)::value;
            constexpr eqtp_gen::CgTerm tm = O2::term(q);
            const float cx = tm.c * in.xv[j][tm.mu1];
            s2 = O2::first(q) ? cx * gj[tm.mu3] : fmaf(cx, gj[tm.mu3], s2);
            if constexpr (O2::last(q)) {
              dy[tm.mu2] = fmaf(wreg[j][tm.p], s2, dy[tm.mu2]);
              __builtin_amdgcn_sched_barrier(0);
            }
          });
        }
      }
      // grad_vec: sum dL/dY over the group's channels (its CL lanes)
#pragma unroll
      for (int off = 1; off < Cfg::CL; off <<= 1)
#pragma unroll
        for (int k = 0; k < K; ++k) dy[k] += __shfl_xor(dy[k], off);
      if (valid && cl == 0) {
        float Y2[16], Gm[16][3];
        sh_grad_eval<L>(in.vx, in.vy, in.vz, Y2, Gm);
        float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
          a0 = fmaf(dy[k], Gm[k][0], a0);
          a1 = fmaf(dy[k], Gm[k][1], a1);
          a2 = fmaf(dy[k], Gm[k][2], a2);
        }
        gvec[3 * (size_t)e] = a0;
        gvec[3 * (size_t)e + 1] = a1;
        gvec[3 * (size_t)e + 2] = a2;
      }
    }
  };

  // wave-uniform rounds over [e_first, e_last); the next round's inputs are
  // fetched before the current round's arithmetic
  auto walk = [&](int e_first, int e_last) {
    EdgeIn cur = fetch(e_first + g, e_first + g < e_last, e_first);
    for (int e0 = e_first; e0 < e_last; e0 += Cfg::G) {
      const int e = e0 + g;
      const EdgeIn nxt = fetch(e + Cfg::G, e + Cfg::G < e_last, e_first);
      round(e, e < e_last, cur);
      cur = nxt;
    }
  };

  if constexpr (SORTED) {
    const int row = blockIdx.x * Cfg::WAVES + wv;
    if (row >= N) return;
    int e_beg = 0, e_end = 0;
    if (E > 0) {
      e_beg = min(max(row_ptr[row], 0), E);
      e_end = min(max(row_ptr[row + 1], e_beg), E);
    }
    if (e_beg == e_end) return;
    load_g(row);
    walk(e_beg, e_end);
  } else {
    const long long base = ((long long)blockIdx.x * Cfg::WAVES + wv) * Cfg::EPW;
    if (base >= E) return;
    walk((int)base, (int)min((long long)E, base + Cfg::EPW));
  }
  // grad_w: combine the lane groups, then one atomic per (path, channel)
  if (PASS == 1 && gw != nullptr) {
#pragma unroll
    for (int off = Cfg::CL; off < kWave; off <<= 1)
#pragma unroll
      for (int j = 0; j < Cfg::CPL; ++j)
#pragma unroll
        for (int p = 0; p < (PASS == 1 ? P : 1); ++p) gwacc[j][p] += __shfl_xor(gwacc[j][p], off);
    if (g == 0) {
#pragma unroll
      for (int j = 0; j < Cfg::CPL; ++j)
#pragma unroll
        for (int p = 0; p < (PASS == 1 ? P : 1); ++p) unsafeAtomicAdd(gw + p * C + cl + j * Cfg::CL, gwacc[j][p]);
    }
  }
}

// ---------------------------------------------------------------------------
// grad_vec of dst-sorted rows on the matrix cores.  For the row of node d and
// an edge e of it, with B_d[c,m1,m2] = sum_p w[p,c] sum_m3 C^p[m1,m2,m3] g[d,c,m3]
// (edge independent):
//   dL/dY_e[m2] = sum_{c,m1} x[src_e,c,m1] B_d[c,m1,m2]
// -- a [16 edges x 256] x [256 x 16] product per 16-channel block on
// v_mfma_f32_16x16x4_f32 (rows = edges, columns = m2, k = (channel, m1)),
// 4 MFMAs per edge and block as in the forward.  One wave per row (persistent
// over rows); per chunk of up to 64 edges and per channel block:
//   1. lanes 0..15 (one channel each) build B_d in LDS from g[d] with the
//      coupling walked in (m1, m2, p) order (runs over m3);
//   2. 16-edge steps: lane (edge i = lane % 16, group kq = lane / 16) loads
//      x[src_i, c, 4kq .. 4kq+3] for the block's 16 channels and feeds the
//      MFMAs; dL/dY accumulates across blocks in registers;
// then dL/dY goes through LDS to one lane per edge, which applies the
// harmonics' Jacobian (sh_grad_eval) and writes grad_vec.
// ---------------------------------------------------------------------------
template <int L, int PS>
struct TermOrderB {  // stable counting sort of the coupling by (mu1, mu2, p)
  using T = Tables<L, PS>;
  struct Idx {
    short v[T::NT];
  };
  static constexpr int key(int i) { return (T::by_out[i].mu1 * 16 + T::by_out[i].mu2) * 64 + T::by_out[i].p; }
  static constexpr int pair(int i) { return T::by_out[i].mu1 * 16 + T::by_out[i].mu2; }
  static constexpr Idx make() {
    Idx a{};
    int pos[16 * 16 * 64 + 1] = {};
    for (int i = 0; i < T::NT; ++i) pos[key(i) + 1]++;
    for (int k = 0; k < 16 * 16 * 64; ++k) pos[k + 1] += pos[k];
    for (int i = 0; i < T::NT; ++i) a.v[pos[key(i)]++] = (short)i;
    return a;
  }
  static constexpr Idx order = make();
  static constexpr const eqtp_gen::CgTerm& term(int j) { return T::by_out[order.v[j]]; }
  static constexpr bool run_first(int j) { return j == 0 || key(order.v[j - 1]) != key(order.v[j]); }
  static constexpr bool run_last(int j) { return j + 1 == T::NT || key(order.v[j + 1]) != key(order.v[j]); }
  static constexpr bool pair_first(int j) { return j == 0 || pair(order.v[j - 1]) != pair(order.v[j]); }
  static constexpr bool pair_last(int j) { return j + 1 == T::NT || pair(order.v[j + 1]) != pair(order.v[j]); }
  // the run that ends at j is the first run of its (mu1, mu2) pair
  static constexpr bool run_opens_pair(int j) {
    while (j > 0 && key(order.v[j - 1]) == key(order.v[j])) --j;
    return pair_first(j);
  }
};

constexpr int kGvBS = 16 * 16 + 4;  // B row per channel (floats): 16-byte rows, stride 4 (mod 64) banks

// slot of row m1 in a channel's B block: rows 4kq + r are rotated by kq within
// their group of four so that the 16-edge steps' reads (fixed r, kq = 0..3)
// hit four different 16-bank groups
__device__ __forceinline__ int gv_slot(int m1) { return (m1 & ~3) | (((m1 & 3) + (m1 >> 2)) & 3); }

template <int L, int PS, int C>
__global__ __launch_bounds__(64) void gvec_node_kernel(int N, int E, const int* __restrict__ row_ptr,
                                                       const float* __restrict__ vec, const int* __restrict__ src,
                                                       const float* __restrict__ x, const float* __restrict__ w,
                                                       const float* __restrict__ gout, float* __restrict__ gvec) {
  using T = Tables<L, PS>;
  using O = TermOrderB<L, PS>;
  constexpr int K = num_comp(L);
  constexpr int CW = C >= 16 ? 16 : C;  // channels per block
  constexpr int NBLK = C / CW;
  __shared__ __attribute__((aligned(16))) float Bl[16 * kGvBS];  // B of one block; then dL/dY [64][17]
  __shared__ int sstg[64];
  const int lane = threadIdx.x & 63;
  const int i16 = lane & 15;
  const int kq = lane >> 4;
  for (int row = blockIdx.x; row < N; row += gridDim.x) {
    int e_beg = 0, e_end = 0;
    if (E > 0) {
      e_beg = min(max(row_ptr[row], 0), E);
      e_end = min(max(row_ptr[row + 1], e_beg), E);
    }
    for (int cb = e_beg; cb < e_end; cb += 64) {
      const int cnt = min(64, e_end - cb);
      // stage the chunk: lane i = edge cb + i
      const bool mine = lane < cnt;
      const int em = mine ? cb + lane : cb;
      const float vx = vec[3 * (size_t)em], vy = vec[3 * (size_t)em + 1], vz = vec[3 * (size_t)em + 2];
      sstg[lane] = mine ? clamp_index(src[em], N) : -1;
      f4 acc[4];
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) acc[s4] = f4{0.f, 0.f, 0.f, 0.f};
      for (int blk = 0; blk < NBLK; ++blk) {
        // x[src] of the edges of 16-edge step s4 for this block: lane (edge i16, group kq) holds
        // components 4kq .. 4kq+3 of the block's 16 channels
        f4 xv[16];
        auto load_step = [&](int s4) {
          const int sv = sstg[16 * s4 + i16];
          const bool ok = sv >= 0;
#pragma unroll
          for (int c = 0; c < 16; ++c) {
            const bool cok = ok && c < CW;
            const size_t o = ((size_t)(cok ? sv : 0) * C + blk * CW + (c < CW ? c : 0)) * K;
            if constexpr (K == 16) {
              xv[c] = cok ? *reinterpret_cast<const f4*>(x + o + 4 * kq) : f4{0.f, 0.f, 0.f, 0.f};
            } else {
#pragma unroll
              for (int r = 0; r < 4; ++r) xv[c][r] = (cok && 4 * kq + r < K) ? x[o + 4 * kq + r] : 0.0f;
            }
          }
        };
        wave_lds_sync();  // previous block's reads of Bl are done; sstg is written
        // the first step's gathers go out before the B_d build, which hides their latency
        load_step(0);
        // 1. B_d for this block's channels (all 16 rows zeroed first: rows of
        //    channels past C stay zero, so the padded MFMA columns add nothing)
        float* brow = Bl + i16 * kGvBS;
        if (lane < 16) {
#pragma unroll
          for (int q = 0; q < 64; ++q) reinterpret_cast<f4*>(brow)[q] = f4{0.f, 0.f, 0.f, 0.f};
        }
        if (lane < CW) {
          const int c = blk * CW + lane;
          float gv[16];
#pragma unroll
          for (int k = 0; k < 16; ++k) gv[k] = k < K ? gout[((size_t)row * C + c) * K + k] : 0.0f;
          float wr[T::P];
#pragma unroll
          for (int p = 0; p < T::P; ++p) wr[p] = w[p * C + c];
          float t = 0.0f, b = 0.0f;
          static_for<0, T::NT>([&](auto jj) {
            constexpr int j = decltype(jj)::value;
            constexpr eqtp_gen::CgTerm tm = O::term(j);
            t = O::run_first(j) ? tm.c * gv[tm.mu3] : fmaf(tm.c, gv[tm.mu3], t);
            if constexpr (O::run_last(j)) b = O::run_opens_pair(j) ? wr[tm.p] * t : fmaf(wr[tm.p], t, b);
            if constexpr (O::pair_last(j)) brow[gv_slot(tm.mu1) * 16 + tm.mu2] = b;
          });
        }
        wave_lds_sync();
        // 2. dL/dY for the chunk's 16-edge steps
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          if (16 * s4 < cnt) {  // wave-uniform
            if (s4 > 0) load_step(s4);
#pragma unroll
            for (int c = 0; c < 16; ++c)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float bv = Bl[c * kGvBS + gv_slot(4 * kq + r) * 16 + i16];
                acc[s4] = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[c][r], bv, acc[s4], 0, 0, 0);
              }
          }
        }
      }
      // 3. dL/dY -> LDS [edge][17]; lane i applies the Jacobian of edge cb + i
      wave_lds_sync();
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
        for (int v = 0; v < 4; ++v) Bl[(16 * s4 + 4 * kq + v) * 17 + i16] = acc[s4][v];
      wave_lds_sync();
      if (mine) {
        float Y2[16], Gm[16][3];
        sh_grad_eval<L>(vx, vy, vz, Y2, Gm);
        float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) {
          const float d = Bl[lane * 17 + k];
          a0 = fmaf(d, Gm[k][0], a0);
          a1 = fmaf(d, Gm[k][1], a1);
          a2 = fmaf(d, Gm[k][2], a2);
        }
        gvec[3 * (size_t)em] = a0;
        gvec[3 * (size_t)em + 1] = a1;
        gvec[3 * (size_t)em + 2] = a2;
      }
    }
  }
}

template <int L, int PS, int C>
static hipError_t launch_bwd_t(const BwdArgs& a) {
  using Cfg = BwdCfg<C>;
  constexpr int K = num_comp(L);
  hipError_t err;
  if (a.gx && a.N > 0 && (err = launch_fill_zero(a.gx, a.N * C * K, a.stream)) != hipSuccess) return err;
  if (a.gw && (err = launch_fill_zero(a.gw, (int64_t)Tables<L, PS>::P * C, a.stream)) != hipSuccess) return err;
  if (a.gvec && a.E > 0 && (err = launch_fill_zero(a.gvec, a.E * 3, a.stream)) != hipSuccess) return err;
  if (a.N == 0 || a.E == 0) return hipSuccess;
  const bool sorted = a.row_ptr != nullptr;
  const long long per_block = (long long)Cfg::WAVES * Cfg::EPW;
  const unsigned blocks = sorted ? (unsigned)((a.N + Cfg::WAVES - 1) / Cfg::WAVES)
                                 : (unsigned)((a.E + per_block - 1) / per_block);
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(blocks), dim3(Cfg::THREADS), 0, a.stream, (int)a.N, (int)a.E, a.row_ptr, a.vec,
                       a.src, a.dst, a.x, a.w, a.gout, a.gx, a.gw, a.gvec);
  };
  if (a.gx != nullptr || a.gw != nullptr) {
    if (sorted) go(conv_bwd_kernel<L, PS, C, true, 1>);
    else go(conv_bwd_kernel<L, PS, C, false, 1>);
  }
  if (a.gvec != nullptr) {
    if (sorted && a.algo != 2) {  // matrix cores unless the vector-ALU walk is asked for
      // one single-wave workgroup per row (the kernel also walks rows persistently for a smaller grid):
      // the dispatcher keeps as many resident as registers and LDS allow (9 per CU) and balances rows
      // of different lengths
      const int64_t g = (int64_t)1 << 24;
      hipLaunchKernelGGL((gvec_node_kernel<L, PS, C>), dim3((unsigned)(a.N < g ? a.N : g)), dim3(64), 0, a.stream,
                         (int)a.N, (int)a.E, a.row_ptr, a.vec, a.src, a.x, a.w, a.gout, a.gvec);
    } else if (sorted) {
      go(conv_bwd_kernel<L, PS, C, true, 2>);
    } else {
      go(conv_bwd_kernel<L, PS, C, false, 2>);
    }
  }
  return hipGetLastError();
}

template <int L, int PS>
static hipError_t dispatch_bwd_c(const BwdArgs& a) {
  switch (a.C) {
    case 8: return launch_bwd_t<L, PS, 8>(a);
    case 16: return launch_bwd_t<L, PS, 16>(a);
    case 32: return launch_bwd_t<L, PS, 32>(a);
    case 64: return launch_bwd_t<L, PS, 64>(a);
    case 128: return launch_bwd_t<L, PS, 128>(a);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_conv_backward(const BwdArgs& a) {
  switch (a.lmax * 2 + a.path_set) {
    case 0: return dispatch_bwd_c<0, 0>(a);
    case 1: return dispatch_bwd_c<0, 1>(a);
    case 2: return dispatch_bwd_c<1, 0>(a);
    case 3: return dispatch_bwd_c<1, 1>(a);
    case 4: return dispatch_bwd_c<2, 0>(a);
    case 5: return dispatch_bwd_c<2, 1>(a);
    case 6: return dispatch_bwd_c<3, 0>(a);
    case 7: return dispatch_bwd_c<3, 1>(a);
    default: return hipErrorInvalidValue;
  }
}

// The radial basis and its derivative in r:
//   dR_n/dr = (a cos(a r) - sin(a r)/r) / r * u + sin(a r)/r * u'(d) / r_c,  a = n pi / r_c,
// with u'(d) = -168 d^5 + 336 d^6 - 168 d^7.  For a r < 1/2 the first term's
// difference of nearly equal quotients is replaced by its Taylor series
// -a^3 r / 3 (1 - t/10 + t^2/280 - t^3/15120), t = (a r)^2 (truncation below
// 3e-9 relative there).  Zero for d >= 1 and at r = 0.
template <int NB>
__device__ __forceinline__ void radial_basis_grad(float r, float inv_rc, float (&R)[NB], float (&dR)[NB]) {
  // branch-free (selects only): early returns that fill the arrays on several paths make the
  // compiler keep them in private memory
  const float d = r * inv_rc;
  const bool inside = d < 1.0f, at_zero = r == 0.0f;
  const float d2 = d * d, d4 = d2 * d2, d6 = d4 * d2;
  const float env = 1.0f + d6 * (-28.0f + d * (48.0f - 21.0f * d));
  const float denv = d4 * d * (-168.0f + d * (336.0f - 168.0f * d)) * inv_rc;  // du/dr
  const float theta = eqtp_gen::kPiF * (inside ? d : 0.0f);  // in [0, pi)
  // sin and cos of theta from their Taylor series on [0, pi/2] (terms to u^13 and u^14, truncation
  // below 3e-8), folded by sin(pi - u) = sin u, cos(pi - u) = -cos u
  const bool upper = theta > 0.5f * eqtp_gen::kPiF;
  const float u = upper ? eqtp_gen::kPiF - theta : theta, u2 = u * u;
  const float s1 =
      u * (1.0f + u2 * (-1.0f / 6 + u2 * (1.0f / 120 + u2 * (-1.0f / 5040 + u2 * (1.0f / 362880 +
          u2 * (-1.0f / 39916800 + u2 * (1.0f / 6227020800.0f)))))));
  const float cu =
      1.0f + u2 * (-0.5f + u2 * (1.0f / 24 + u2 * (-1.0f / 720 + u2 * (1.0f / 40320 + u2 * (-1.0f / 3628800 +
          u2 * (1.0f / 479001600 - u2 * (1.0f / 87178291200.0f)))))));
  const float c1 = upper ? -cu : cu;
  const float inv_r = at_zero ? 0.0f : 1.0f / r;
  float sm1 = 0.0f, s = s1, cm1 = 1.0f, c = c1;  // sin, cos of n theta by the Chebyshev recurrence
  const float c2 = 2.0f * c1;
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    const float a = (float)(n + 1) * eqtp_gen::kPiF * inv_rc;
    const float ar = (float)(n + 1) * theta;
    const float f = at_zero ? a : s * inv_r;  // sin(a r) / r, its limit a at r = 0
    const float t = ar * ar;
    const float series = -(a * a * a * r) * (1.0f / 3.0f) *
                         (1.0f + t * (-0.1f + t * (1.0f / 280.0f - t * (1.0f / 15120.0f))));
    const float df = ar < 0.5f ? series : (a * c - f) * inv_r;
    R[n] = inside ? f * env : 0.0f;
    dR[n] = inside ? df * env + f * denv : 0.0f;
    const float sn = c2 * s - sm1, cn = c2 * c - cm1;
    sm1 = s;
    s = sn;
    cm1 = c;
    c = cn;
  }
}

// ---------------------------------------------------------------------------
// Gradients with radial weights, w_e[p,c] = sum_b R_b(r_e) W[b, p*C + c]
// (the radial basis above, 8 functions; r_e = |vec_e|).  Per edge e = (s -> d)
// and channel c, in the edge frame (the edge-aligned form of the coupling,
// E2Former-V2 page, section 2.1): with D = D(R_e), x' = D x[s], g' = D g[d]
// and P_p the sparse coupling of path p at the frame's pole,
//   v' = sum_p w_e[p,c] P_p^T g',  grad_x[s,c] += D^T v'
//   T_e[p,c] = g' . P_p x'                                  (dL/dw_e[p,c])
//   grad_W[b,p*C+c] += R_b(r_e) T_e[p,c]
//   dL/dr_e += sum_b R_b'(r_e) sum_p W[b,p*C+c] T_e[p,c]
//   u' = sum_p w_e[p,c] P_p x',  G_x = -(v' . L_y x' + u' . L_y g'),
//   G_y = v' . L_x x' + u' . L_x g'  (the harmonics' part, by the rotation
//   generators; so2_device.hpp, gen_form)
//   grad_vec[e] = R_e^T (G_x, G_y, 0) / r_e + dL/dr_e vec_e / r_e.
// Lane layout: a workgroup works on one block of 16 channels (lane j of each
// 16-lane group), its four waves on edges of their own (sorted: one row per
// wave, rows strided over the block's workgroups; unsorted: runs of 64 edges),
// four edges per round (lane group kq takes edge kq).  The block's slice of W
// sits in LDS as [p][j][b] (two 16-byte reads give a lane the 8 weights of a
// path), read one path ahead of its use.
// One walk of the sparse terms by (path, mu3) runs gives v', u' and T_p; per
// path the lane keeps (sum_b R_b' W_b) T_p for dL/dr and stages T_p in LDS.
// After the walk, per path, D[b][j] = sum_kq R_b(edge kq) T_p(edge kq, j) is
// one v_mfma_f32_16x16x4_f32 (A rows = b, 8 of 16 used; k = the round's four
// edges; B = the staged T_p), accumulated in the wave's matrix-core result
// registers over its whole run of edges; the sums go into an LDS copy of the
// block's grad_W slice once per wave and to memory once per workgroup.  grad_x
// goes out as in the fixed-weight walk (the round's 4 x 16 x K contributions
// through LDS, 64 contiguous floats per atomic instruction); grad_vec is
// reduced over the block's 16 channels and added with fp32 atomics (one per
// block and component).  Lanes of a round past the last edge load an in-range
// edge and zero its radial functions, which zeroes all their contributions.
// The walk is kept free of branches, and the running sums of each path are
// settled (an empty asm that takes them as operands) before the next path
// starts: otherwise the compiler is free to leave sums to the end of the walk
// with all their inputs live, several hundred registers at lmax 3.
// ---------------------------------------------------------------------------
// true if the edge-aligned terms hold every path 0..P-1, in path order (the walk below reads the next
// path's weights one path ahead)
template <class S>
constexpr bool so2_paths_in_order() {
  int expect = 0;
  for (int i = 0; i < S::NT; ++i) {
    if (S::terms[i].p == expect) ++expect;
    else if (S::terms[i].p != expect - 1) return false;
  }
  return expect == S::P;
}

constexpr int kRbNB = 8;     // radial functions
constexpr int kRbWaves = 4;  // waves per workgroup
constexpr int kRbChunk = 64; // edges per run, unsorted edges

// MODE 0: edges in any order (runs of kRbChunk; src, dst per edge); 1: dst-sorted (row_ptr over
// destinations, src per edge); 2: grouped by source (row_ptr over sources, dst per edge, perm[i] = the
// input index of grouped edge i for grad_vec): grad_x is summed per source row in LDS and written once.
template <int L, int PS, int MODE>
__global__ __launch_bounds__(kRbWaves * kWave) void conv_bwd_radial_kernel(
    int N, int E, int C, int nwg, const int* __restrict__ row_ptr, const float* __restrict__ vec,
    const int* __restrict__ src, const int* __restrict__ dst, const int* __restrict__ perm,
    const float* __restrict__ x, const float* __restrict__ W, const float* __restrict__ gout,
    float* __restrict__ gx, float* __restrict__ gW, float* __restrict__ gvec, float inv_rc) {
  using T = Tables<L, PS>;
  using S = So2Tables<L, PS>;
  constexpr int K = num_comp(L);
  constexpr int P = T::P;
  constexpr int NB = kRbNB;
  static_assert(S::P == P && so2_paths_in_order<S>(), "edge-aligned terms: every path, in path order");
  constexpr int XB = 16 * K;  // floats of one edge's block of 16 channels
  __shared__ __attribute__((aligned(16))) float wt[P * 16 * NB];  // W slice, [p][j][b]
  constexpr int GWL = NB * P * 16;
  __shared__ float gwl[GWL];  // grad_W slice, [b][p][j]
  // per wave: the round's T_p (P x 64) during the walk, then its grad_x exchange (4 x XB)
  constexpr int XCH = 64 * P > 4 * XB ? 64 * P : 4 * XB;
  __shared__ __attribute__((aligned(16))) float xch[kRbWaves][XCH];
  __shared__ int xsrc[kRbWaves][4];
  // grouped by source: the row's grad_x sums, lane (kq, j) owning floats (kq * 16 + j) * K .. + K - 1
  __shared__ __attribute__((aligned(16))) float gxa[kRbWaves][MODE == 2 ? 4 * XB : 1];
  const int cb = (int)(blockIdx.x / nwg) * 16;
  const int wg = (int)(blockIdx.x % nwg);
  for (int i = threadIdx.x; i < P * 16 * NB; i += kRbWaves * kWave) {
    const int b = i % NB, jj = (i / NB) % 16, p = i / (NB * 16);
    wt[i] = W[(size_t)b * P * C + (size_t)p * C + cb + jj];
    gwl[i] = 0.0f;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int j = lane & 15;   // channel cb + j
  const int kq = lane >> 4;  // edge of the round
  const bool want_x = gx != nullptr, want_w = gW != nullptr;
  const bool want_v = gvec != nullptr;
  float* const xw = xch[wv];
  // the wave's grad_W sums, D_p[b][j] of path p in lane (j, rows 4 kq .. 4 kq + 3), b < 8 in lanes < 32
  f4 gacc[P];
#pragma unroll
  for (int p = 0; p < P; ++p) gacc[p] = f4{0.f, 0.f, 0.f, 0.f};

  // one round: lane group kq takes edge e (valid) or, if past the end, edge e_alt with no weight
  auto round = [&](int e, bool valid, int e_alt, int row) {
    const int ec = valid ? e : e_alt;
    const float vx = vec[3 * (size_t)ec], vy = vec[3 * (size_t)ec + 1], vz = vec[3 * (size_t)ec + 2];
    // the row's node (dst-sorted: the destination, grouped by source: the source) is read again each
    // round from the cache rather than held in registers across the row
    int s = MODE == 2 ? row : clamp_index(src[ec], N);
    if constexpr (MODE == 2) asm volatile("" : "+v"(s));  // a new value each round: not hoisted out of the row
    float xv[K], gv[K];
#pragma unroll
    for (int k = 0; k < K; ++k) xv[k] = x[((size_t)s * C + cb + j) * K + k];
    int d = MODE == 1 ? row : clamp_index(dst[ec], N);
    if constexpr (MODE == 1) asm volatile("" : "+v"(d));
#pragma unroll
    for (int k = 0; k < K; ++k) gv[k] = gout[((size_t)d * C + cb + j) * K + k];
    const float r = sqrtf(vx * vx + vy * vy + vz * vz);
    float R[NB], dR[NB];
    radial_basis_grad<NB>(r, inv_rc, R, dR);
    if (!valid) {
#pragma unroll
      for (int b = 0; b < NB; ++b) R[b] = dR[b] = 0.0f;
    }
    float g0 = 0.0f, g1 = 0.0f, g2 = 0.0f;  // this lane's part of grad_vec
    // The lane's 8 weights of path p are read from LDS one path ahead.  The offset of each read passes
    // through an empty asm that takes the previous path's w_p as input: the read can then not be issued
    // before that path starts, so at most two paths' weights are held in registers at a time (the
    // compiler would otherwise issue all 2 P reads up front).
    int woff = j * NB;
    asm volatile("" : "+v"(woff));
    f4 nlo = reinterpret_cast<const f4*>(wt + woff)[0], nhi = reinterpret_cast<const f4*>(wt + woff)[1];
    auto settle = [&](float (&v)[K]) {
#pragma unroll
      for (int k = 0; k < K; ++k) asm volatile("" : "+v"(v[k]));
    };
    auto prefetch = [&](int p_next, float after, float& settle) {
      // settle: a running sum that must be complete here (else the compiler may leave its terms, and
      // their inputs, live until the end of the walk)
      asm volatile("" : "+v"(woff), "+v"(settle) : "v"(after));
      const f4* wr = reinterpret_cast<const f4*>(wt + p_next * 16 * NB + woff);
      nlo = wr[0];
      nhi = wr[1];
    };

    {
      float aR = 0.0f;  // MFMA A operand: R_j of this lane's edge (rows j >= 8 are zero)
#pragma unroll
      for (int b = 0; b < NB; ++b) aR = j == b ? R[b] : aR;
      // The walk in the edge frame (the edge-aligned form of the coupling): with D = D(R_e),
      // message_e = D^T P(w_e) D x, so grad_x = D^T P(w_e)^T D g and T_p = (D g) . P_p (D x); x and g are
      // rotated in, the sparse terms (by (path, mu3) runs) give both, the grad_x sums are rotated back.
      const So2Frame<L> fr(vx, vy, vz);
      float xr[K], gr[K], mx[K], ux[K];  // mx: v' = P_w^T g' (grad_x in the frame); ux: u' = P_w x'
#pragma unroll
      for (int k = 0; k < K; ++k) {
        xr[k] = xv[k];
        gr[k] = gv[k];
        mx[k] = 0.0f;
        ux[k] = 0.0f;
      }
      so2_rotate_in<L>(xr, fr);
      so2_rotate_in<L>(gr, fr);
      // wp = sum_b R_b W_b (the path weight), wd = sum_b R_b' W_b (its derivative in r)
      float wp = 0.0f, wd = 0.0f, tp = 0.0f, t = 0.0f, qg = 0.0f, dr = 0.0f;
      static_for<0, S::NT>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
        constexpr eqtp_gen::So2Term tm = S::terms[i];
        constexpr bool p_first = i == 0 || S::terms[i - 1].p != tm.p;
        constexpr bool p_last = i + 1 == S::NT || S::terms[i + 1].p != tm.p;
        constexpr bool run_first = p_first || S::terms[i - 1].mu3 != tm.mu3;
        constexpr bool run_last = p_last || S::terms[i + 1].mu3 != tm.mu3;
        if constexpr (p_first) {
          wp = wd = 0.0f;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            wp = fmaf(R[b], nlo[b], wp);
            wp = fmaf(R[4 + b], nhi[b], wp);
            wd = fmaf(dR[b], nlo[b], wd);
            wd = fmaf(dR[4 + b], nhi[b], wd);
          }
          if constexpr (tm.p + 1 < P) {
            prefetch(tm.p + 1, wp, dr);
            settle(mx);  // likewise the grad_x sums: each path's terms are added before the next starts
            settle(ux);
          }
          if constexpr (tm.l2 > 0) wp *= fr.keep;  // a zero vector drops the paths with l2 > 0
          tp = 0.0f;
        }
        if constexpr (run_first) qg = wp * gr[tm.mu3];
        mx[tm.mu1] = fmaf(tm.c, qg, mx[tm.mu1]);
        t = run_first ? tm.c * xr[tm.mu1] : fmaf(tm.c, xr[tm.mu1], t);
        if constexpr (run_last) {
          tp = fmaf(gr[tm.mu3], t, tp);
          ux[tm.mu3] = fmaf(wp, t, ux[tm.mu3]);
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (p_last) {
          // (no branches in the walk: a branch per path splits it into blocks across which the compiler
          // keeps common products live)
          if constexpr (tm.l2 > 0) tp *= fr.keep;
          dr = fmaf(wd, tp, dr);                // dL/dr += sum_b R_b' W_b T_p
          xw[tm.p * kWave + lane] = tp;         // T_p of the round, for the grad_W products below
          __builtin_amdgcn_sched_barrier(0);
        }
      });
      // the harmonics' part of grad_vec, in the frame: the generators of rotations about its x and y
      // axes act on the rotated features (so2_device.hpp, gen_form); with dL/dr, along vec / r below
      float ga0 = 0.0f, ga1 = 0.0f, ga2 = 0.0f;
      if (want_v && r > 0.0f) {
        __builtin_amdgcn_sched_barrier(0);
        const float gxe = -(gen_form<K, false>(mx, xr) + gen_form<K, false>(ux, gr));
        __builtin_amdgcn_sched_barrier(0);
        const float gye = gen_form<K, true>(mx, xr) + gen_form<K, true>(ux, gr);
        __builtin_amdgcn_sched_barrier(0);
        frame_gradient<L>(fr, gxe, gye, 1.0f / r, ga0, ga1, ga2);
      }
      so2_rotate_out<L>(mx, fr);
      if (want_w) {
        // grad_W: per path, D[b][j] += sum_kq R_b(edge kq) T_p(edge kq, j) on the matrix cores, into the
        // wave's accumulators
        wave_lds_sync();
        static_for<0, P>([&](auto pp) {
          constexpr int p = decltype(pp)::value;
          gacc[p] = __builtin_amdgcn_mfma_f32_16x16x4f32(aR, xw[p * kWave + lane], gacc[p], 0, 0, 0);
        });
        wave_lds_sync();
      }
      if (MODE == 2 && want_x) {  // grouped by source: into the row's sums (lane-private slots)
        float* const ga = gxa[wv] + (kq * 16 + j) * K;
#pragma unroll
        for (int k = 0; k < K; ++k) ga[k] += mx[k];
      } else if (want_x) {
#pragma unroll
        for (int k = 0; k < K; ++k) xw[(kq * 16 + j) * K + k] = mx[k];
        if (j == 0) xsrc[wv][kq] = valid ? s : -1;
        wave_lds_sync();
#pragma unroll
        for (int t = 0; t < K; ++t) {  // 4 * XB floats = K instructions of 64
          const int f = kWave * t + lane;
          const int sd = xsrc[wv][f / XB];
          if (sd >= 0) unsafeAtomicAdd(gx + ((size_t)sd * C + cb) * K + f % XB, xw[f]);
        }
        wave_lds_sync();
      }
      if (want_v && r > 0.0f) {  // the radial part: dL/dr along vec / r
        const float qr = dr / r;
        g0 = fmaf(qr, vx, ga0);
        g1 = fmaf(qr, vy, ga1);
        g2 = fmaf(qr, vz, ga2);
      }
    }
    if (want_v) {  // the block's 16 channels, then one atomic per component
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        g0 += __shfl_xor(g0, off);
        g1 += __shfl_xor(g1, off);
        g2 += __shfl_xor(g2, off);
      }
      if (j == 0 && valid) {
        const size_t ge = MODE == 2 ? (size_t)clamp_index(perm[e], E) : (size_t)e;
        unsafeAtomicAdd(gvec + 3 * ge, g0);
        unsafeAtomicAdd(gvec + 3 * ge + 1, g1);
        unsafeAtomicAdd(gvec + 3 * ge + 2, g2);
      }
    }
  };

  if constexpr (MODE == 1) {
    for (int row = wg * kRbWaves + wv; row < N; row += nwg * kRbWaves) {
      const int e_beg = min(max(row_ptr[row], 0), E);
      const int e_end = min(max(row_ptr[row + 1], e_beg), E);
      for (int e0 = e_beg; e0 < e_end; e0 += 4) round(e0 + kq, e0 + kq < e_end, e_beg, row);
    }
  } else if constexpr (MODE == 2) {
    float* const ga = gxa[wv];
    for (int row = wg * kRbWaves + wv; row < N; row += nwg * kRbWaves) {
      const int e_beg = min(max(row_ptr[row], 0), E);
      const int e_end = min(max(row_ptr[row + 1], e_beg), E);
      if (want_x) {
#pragma unroll
        for (int k = 0; k < K; ++k) ga[(kq * 16 + j) * K + k] = 0.0f;
      }
      for (int e0 = e_beg; e0 < e_end; e0 += 4) round(e0 + kq, e0 + kq < e_end, e_beg, row);
      if (want_x) {  // the four edge groups' sums, one coalesced store of the row's block (zeros if no edges)
        wave_lds_sync();
#pragma unroll
        for (int t = 0; t < (XB + kWave - 1) / kWave; ++t) {
          const int f = kWave * t + lane;  // float f of the block's 16 x K
          if (f < XB) gx[((size_t)row * C + cb) * K + f] = ga[f] + ga[XB + f] + ga[2 * XB + f] + ga[3 * XB + f];
        }
        wave_lds_sync();
      }
    }
  } else {
    const int nchunk = (E + kRbChunk - 1) / kRbChunk;
    for (int ch = wg * kRbWaves + wv; ch < nchunk; ch += nwg * kRbWaves) {
      const int e_first = ch * kRbChunk;
      const int e_last = min(E, e_first + kRbChunk);
      for (int e0 = e_first; e0 < e_last; e0 += 4) round(e0 + kq, e0 + kq < e_last, e_first, 0);
    }
  }
  {
    if (want_w && lane < 32) {  // the wave's sums into the workgroup's slice (rows b = 4 kq + r < 8)
#pragma unroll
      for (int p = 0; p < P; ++p)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          __hip_atomic_fetch_add(&gwl[((4 * kq + rr) * P + p) * 16 + j], gacc[p][rr], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
  __syncthreads();
  if (want_w) {
    for (int i = threadIdx.x; i < GWL; i += kRbWaves * kWave) {
      const int b = i / (P * 16), p = (i / 16) % P, jj = i % 16;
      unsafeAtomicAdd(gW + (size_t)b * P * C + (size_t)p * C + cb + jj, gwl[i]);
    }
  }
}

template <int L, int PS>
static hipError_t launch_bwd_radial_t(const BwdArgs& a) {
  constexpr int K = num_comp(L);
  constexpr int P = Tables<L, PS>::P;
  hipError_t err;
  // grouped by source every row's grad_x block is written once; else it is a sum of atomics
  if (a.gx && a.N > 0 && !a.by_src && (err = launch_fill_zero(a.gx, a.N * a.C * K, a.stream)) != hipSuccess)
    return err;
  if (a.gw && (err = launch_fill_zero(a.gw, (int64_t)kRbNB * P * a.C, a.stream)) != hipSuccess) return err;
  if (a.gvec && a.E > 0 && (err = launch_fill_zero(a.gvec, a.E * 3, a.stream)) != hipSuccess) return err;
  if (a.N > 0 && a.E == 0 && a.by_src && a.gx &&
      (err = launch_fill_zero(a.gx, a.N * a.C * K, a.stream)) != hipSuccess)
    return err;
  if (a.N == 0 || a.E == 0) return hipSuccess;
  const bool sorted = a.row_ptr != nullptr;
  const int nblk = a.C / 16;
  // about four resident workgroups per CU over the whole grid; each wave walks rows or runs strided
  const int64_t units = sorted ? a.N : (a.E + kRbChunk - 1) / kRbChunk;
  const int64_t want = (4LL * num_cus() + nblk - 1) / nblk;
  const int64_t cap = (units + kRbWaves - 1) / kRbWaves;
  const int nwg = (int)(want < cap ? want : cap);
  const unsigned grid = (unsigned)(nblk * nwg);
  const float inv_rc = 1.0f / a.r_cut;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kRbWaves * kWave), 0, a.stream, (int)a.N, (int)a.E, a.C, nwg,
                       a.row_ptr, a.vec, a.src, a.dst, a.perm, a.x, a.w, a.gout, a.gx, a.gw, a.gvec, inv_rc);
  };
  if (a.by_src) go(conv_bwd_radial_kernel<L, PS, 2>);
  else if (sorted) go(conv_bwd_radial_kernel<L, PS, 1>);
  else go(conv_bwd_radial_kernel<L, PS, 0>);
  return hipGetLastError();
}

hipError_t launch_conv_backward_radial(const BwdArgs& a) {
  if (a.C % 16 != 0) return hipErrorInvalidValue;
  switch (a.lmax * 2 + a.path_set) {
    case 0: return launch_bwd_radial_t<0, 0>(a);
    case 1: return launch_bwd_radial_t<0, 1>(a);
    case 2: return launch_bwd_radial_t<1, 0>(a);
    case 3: return launch_bwd_radial_t<1, 1>(a);
    case 4: return launch_bwd_radial_t<2, 0>(a);
    case 5: return launch_bwd_radial_t<2, 1>(a);
    case 6: return launch_bwd_radial_t<3, 0>(a);
    case 7: return launch_bwd_radial_t<3, 1>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace eqtp
