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
// Work decomposition: a task is (destination row, block of 16 channels), run by
// one independent wavefront (a one-wave workgroup); persistent wavefronts walk
// the task list with a stride that keeps each wave on one channel block.
//   * The row's edges are staged 64 at a time: lane i loads edge i's vector
//     and source (coalesced), evaluates its harmonics and writes them, and the
//     byte offset of the source's channel block, to the wave's LDS.
//   * Each 4-edge step: lane l feeds A = Y[edge l/16][mu2 = l%16] and, for
//     each mu1, B = x[src, channel, mu1] from four 16-byte loads per lane
//     (16 lanes cover 4 channels x 16 components = 256 contiguous bytes per
//     edge and load); two steps of loads are kept in flight.
//   * After the row, G goes to LDS (rows laid out so that the stores are free
//     of bank conflicts) and lanes 0..15 (= channels) run the whole coupling
//     with the coefficients as instruction immediates, then store their
//     64-byte output rows.
// The same kernel gives the gradients with respect to x and w (TR = true).
// For L = sum gout * out, with the edges grouped by source node s:
//   H_s[c,mu3,mu2]  = sum_{e: src_e = s} gout[dst_e,c,mu3] * Y_mu2(vec_e)
//   grad_x[s,c,mu1] = sum_p w[p,c] sum_{mu2,mu3} C^p[mu1,mu2,mu3] H_s[c,mu3,mu2]
//   grad_w[p,c]     = sum_s sum_{mu1} x[s,c,mu1] sum_{mu2,mu3} C^p[mu1,mu2,mu3] H_s[c,mu3,mu2]
// H_s is the forward's G with gout gathered through dst instead of x through
// src, and the contraction is the forward's with mu1 and mu3 exchanged
// (AdjointTables); grad_w reuses each run's partial sum with one more FMA.
#include <atomic>

#include "eqtp_device.hpp"
#include "eqtp_kernels.hpp"

namespace eqtp {

// The coupling with the roles of mu1 and mu3 exchanged (C'^p[mu3,mu2,mu1] =
// C^p[mu1,mu2,mu3]), listed by (new mu3, p) so that every (p, mu3) run of the
// contraction below is contiguous.
template <int L, int PS>
struct AdjointTables {
  using B = Tables<L, PS>;
  static constexpr int P = B::P;
  static constexpr int NT = B::NT;
  struct Arr {
    eqtp_gen::CgTerm v[NT];
  };
  static constexpr int key(const eqtp_gen::CgTerm& t) { return t.mu1 * 64 + t.p; }
  static constexpr Arr make() {  // stable counting sort by key
    Arr a{};
    int pos[16 * 64 + 1] = {};
    for (int i = 0; i < NT; ++i) pos[key(B::by_out[i]) + 1]++;
    for (int k = 0; k < 16 * 64; ++k) pos[k + 1] += pos[k];
    for (int i = 0; i < NT; ++i) {
      const eqtp_gen::CgTerm t = B::by_out[i];
      a.v[pos[key(t)]++] = eqtp_gen::CgTerm{t.p, t.mu3, t.mu2, t.mu1, t.c};
    }
    return a;
  }
  static constexpr Arr arr = make();
  static constexpr const eqtp_gen::CgTerm* by_out = arr.v;
};

template <int L, int C>
struct NodeCfg {
  static constexpr int K = num_comp(L);
  static constexpr int CW = C >= 16 ? 16 : C;            // channels per wave (MFMA columns in use)
  static constexpr int NBLK = C / CW;                    // channel blocks per row
  // G row per channel: K*K floats padded to a multiple of 4 (16-byte rows) with
  // stride = 4 (mod 32) words, so 8 lanes' 16-byte accesses hit distinct banks
  static constexpr int GS = ((K * K + 3) / 4 * 4) % 32 == 4 ? (K * K + 3) / 4 * 4
                                                          : ((K * K + 3) / 4 * 4 + 31) / 32 * 32 + 4;
  static constexpr int SLICE = CW * GS;                  // G slice (floats)
  static constexpr int YS = 20;                          // staged Y row stride: 16-byte rows on distinct banks
  static constexpr int STG = 64 * YS + 64;               // staging: Y[64][YS] + src[64]
  // G row of feature component mu1 (K = 16): rows mu1 and mu1 + 4 on opposite bank halves, so that the
  // 16-byte stores of 8 consecutive lanes (4 channels x 2 component groups) hit distinct banks
  static constexpr int grow(int mu1) { return K == 16 ? (mu1 ^ ((mu1 >> 2) & 1)) : mu1; }
  static constexpr int LDS = SLICE > STG ? SLICE : STG;  // staging and G share the wave's LDS
  static constexpr int THREADS = kWave;                  // one independent wavefront per workgroup
  static constexpr int PF = 2;                           // gather steps in flight
  static_assert(LDS * 4 <= 64 * 1024, "LDS budget");
};

// The task schedule shared by the convolution and its test probe.
//   * Task t = (row t / NBLK, channel block t % NBLK); persistent wavefronts
//     take t = blockIdx.x, blockIdx.x + gridDim.x, ...  The next task's CSR
//     bounds and first 64 edges (vector, source) are loaded while the current
//     one runs.
//   * A row's edges are staged 64 at a time (stage(valid, vx, vy, vz, s):
//     lane i holds edge i of the chunk) and consumed in 4-edge steps: lane l
//     takes slot 4*step + l/16.  load(slot, live) issues a step's reads and
//     compute(data) consumes them; PF steps are kept in flight in a ring.
//     Loads are issued unconditionally (steps past the end are "not live" and
//     read nothing), so the wait for a step covers that step's loads only.
//   * task_end(row, blk) runs after each task (the epilogue).
// BUF: edge vectors and sources come through raw buffer loads (< 4 GiB).
template <int PF, int NBLK, bool BUF, class Stage, class Load, class Compute, class TaskEnd>
__device__ __forceinline__ void node_tasks(int N, int E, const int* __restrict__ row_ptr, const float* __restrict__ vec,
                                           const int* __restrict__ src, Stage&& stage, Load&& load,
                                           Compute&& compute, TaskEnd&& task_end) {
  const int lane = threadIdx.x & 63;
  const int kq = lane >> 4;
  const long long ntasks = (long long)N * NBLK;
  const rsrc_t rvec = make_rsrc(vec, vec != nullptr ? (uint64_t)E * 12u : 0u);
  const rsrc_t rsrc = make_rsrc(src, (uint64_t)E * 4u);
  auto bounds = [&](long long t, int& b, int& e) {
    const int r = (int)(t / NBLK);
    b = 0;
    e = 0;
    if (E > 0) {
      b = min(max(row_ptr[r], 0), E);
      e = min(max(row_ptr[r + 1], b), E);
    }
  };
  auto edge_in = [&](int b, int e, int i, float& vx, float& vy, float& vz, int& s, bool& valid) {
    valid = b + i < e;
    if constexpr (BUF) {
      const uint32_t k = valid ? (uint32_t)(b + i) : 0u;
      const uint32_t ov = valid ? 12u * k : kOutOfRange;
      vx = buf_f32(rvec, ov);
      vy = buf_f32(rvec, ov + 4u);
      vz = buf_f32(rvec, ov + 8u);
      s = clamp_index(buf_i32(rsrc, valid ? 4u * k : kOutOfRange), N);
    } else {
      const int k = valid ? b + i : 0;
      vx = vy = vz = 0.0f;
      s = 0;
      if (valid) {
        if (vec != nullptr) {
          vx = vec[3 * (size_t)k];
          vy = vec[3 * (size_t)k + 1];
          vz = vec[3 * (size_t)k + 2];
        }
        s = clamp_index(src[k], N);
      }
    }
  };
  long long t = blockIdx.x;
  if (t >= ntasks) return;
  int e_beg, e_end;
  bounds(t, e_beg, e_end);
  float pvx, pvy, pvz;
  int ps;
  bool pvalid;
  edge_in(e_beg, e_end, lane, pvx, pvy, pvz, ps, pvalid);
  while (true) {
    const long long tn = t + gridDim.x;
    int nb = 0, ne = 0;
    if (tn < ntasks) bounds(tn, nb, ne);
    bool next_loaded = false;
    float qvx = 0.f, qvy = 0.f, qvz = 0.f;
    int qs = 0;
    bool qvalid = false;
    for (int cb = e_beg; cb < e_end; cb += 64) {
      const int cnt = min(64, e_end - cb);
      if (cb != e_beg) edge_in(cb, e_end, lane, pvx, pvy, pvz, ps, pvalid);
      stage(pvalid, pvx, pvy, pvz, ps);
      wave_lds_sync();
      const int nsteps = (cnt + 3) >> 2;
      decltype(load(0, true)) ring[PF];
#pragma unroll
      for (int q = 0; q < PF; ++q) ring[q] = load(4 * min(q, 15) + kq, q < nsteps);
      if (!next_loaded) {
        edge_in(nb, ne, lane, qvx, qvy, qvz, qs, qvalid);
        next_loaded = true;
      }
      for (int base = 0; base < nsteps; base += PF) {
#pragma unroll
        for (int q = 0; q < PF; ++q) {
          if (base + q < nsteps) compute(ring[q]);
          const int st = base + q + PF;
          ring[q] = load(4 * min(st, 15) + kq, st < nsteps);
        }
      }
      wave_lds_sync();
    }
    if (!next_loaded) edge_in(nb, ne, lane, qvx, qvy, qvz, qs, qvalid);
    task_end((int)(t / NBLK), (int)(t % NBLK));
    wave_lds_sync();
    if (tn >= ntasks) break;
    t = tn;
    e_beg = nb;
    e_end = ne;
    pvx = qvx;
    pvy = qvy;
    pvz = qvz;
    ps = qs;
    pvalid = qvalid;
  }
}

// XB: the node features are bfloat16 (widened to fp32 on load: a bf16 value
// is the upper half of the fp32 with the same bits), halving the gather.
// TR: gradients (see the top of the file): rows are source nodes, src holds
// each edge's destination, xp is gout, out receives grad_x (may be null) and
// grad_w (if non-null, zero-filled beforehand) is accumulated from xn = x.
template <int L, int PS, int C, bool BUF, bool XB, bool TR>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void conv_node_kernel(
    int N, int E, const int* __restrict__ row_ptr, const float* __restrict__ vec, const int* __restrict__ src,
    const void* __restrict__ xp, const float* __restrict__ w, float* __restrict__ out, const float* __restrict__ xn,
    float* __restrict__ gw) {
  using Cfg = NodeCfg<L, C>;
  using T = std::conditional_t<TR, AdjointTables<L, PS>, Tables<L, PS>>;
  constexpr int K = Cfg::K;
  __shared__ __attribute__((aligned(16))) float lds[Cfg::LDS];

  const int lane = threadIdx.x & 63;
  float* ystg = lds;
  int* sstg = reinterpret_cast<int*>(lds + 64 * Cfg::YS);
  constexpr uint32_t XS = XB ? 2u : 4u;  // bytes per feature element
  const rsrc_t rx = make_rsrc(xp, (uint64_t)N * C * K * XS);
  const float* const x = static_cast<const float*>(xp);
  const uint16_t* const xh = static_cast<const uint16_t*>(xp);
  // 4 consecutive features from element index i, or 1 (zeros when !v)
  auto ld4 = [&](size_t i, bool v) -> f4 {
    if constexpr (XB) {
      uint32_t d0 = 0, d1 = 0;
      if constexpr (BUF) {
        const auto t = __builtin_amdgcn_raw_buffer_load_b64(rx, v ? (int)(uint32_t)(i * 2) : (int)kOutOfRange, 0, 0);
        d0 = t[0];
        d1 = t[1];
      } else if (v) {
        const uint2 t = *reinterpret_cast<const uint2*>(xh + i);
        d0 = t.x;
        d1 = t.y;
      }
      return f4{__uint_as_float(d0 << 16), __uint_as_float(d0 & 0xffff0000u), __uint_as_float(d1 << 16),
                __uint_as_float(d1 & 0xffff0000u)};
    } else {
      if constexpr (BUF) return buf_f4(rx, v ? (uint32_t)(i * 4) : kOutOfRange);
      else return v ? *reinterpret_cast<const f4*>(x + i) : f4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto ld1 = [&](size_t i, bool v) -> float {
    if constexpr (XB) {
      uint32_t h = 0;
      if constexpr (BUF) h = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rx, v ? (int)(uint32_t)(i * 2) : (int)kOutOfRange, 0, 0);
      else if (v) h = xh[i];
      return __uint_as_float(h << 16);
    } else {
      if constexpr (BUF) return buf_f32(rx, v ? (uint32_t)(i * 4) : kOutOfRange);
      else return v ? x[i] : 0.0f;
    }
  };

  const int cl = lane & 15;  // MFMA column
  const bool c_ok = cl < Cfg::CW;
  // fp32 features in one buffer resource, 16 components, 16-channel blocks: the staging keeps each edge's
  // gather offset (bytes of its source's channel block) instead of its source index
  constexpr bool kOffsets = BUF && !XB && K == 16 && Cfg::CW == 16;

  f4 acc[K];
#pragma unroll
  for (int k = 0; k < K; ++k) acc[k] = f4{0.f, 0.f, 0.f, 0.f};
  // grad_w partial sums, [P][16] (lane = channel within the block); in LDS
  // rather than registers, which the contraction needs
  __shared__ float gwl[TR ? T::P * 16 : 1];
  if constexpr (TR) {
    if (lane < 16) {
#pragma unroll
      for (int p = 0; p < T::P; ++p) gwl[p * 16 + lane] = 0.0f;
    }
  }
  int c_base = (int)(blockIdx.x % Cfg::NBLK) * Cfg::CW;  // first channel of the current task's block

  auto stage = [&](bool valid, float vx, float vy, float vz, int s) {
    float Y[16];
    sh_eval<L>(vx, vy, vz, Y);
    const float m = valid ? 1.0f : 0.0f;  // padding slots contribute nothing
    f4* yd = reinterpret_cast<f4*>(ystg + lane * Cfg::YS);
#pragma unroll
    for (int q = 0; q < 4; ++q) yd[q] = f4{m * Y[4 * q], m * Y[4 * q + 1], m * Y[4 * q + 2], m * Y[4 * q + 3]};
    if constexpr (kOffsets)
      sstg[lane] = valid ? (int)(((uint32_t)s * C + c_base) * K * 4u) : (int)0xFFFFF000u;  // byte offset or out of range
    else
      sstg[lane] = valid ? s : -1;  // -1: the slot's gather reads nothing
  };

  // B operand columns.  K = 16: column n = lane%16 stands for (channel
  // 4j + n%4, components 4(n/4)..4(n/4)+3) of channel group j, so one 16-byte
  // load per lane and j reads 256 contiguous bytes per edge (4 channels x 16
  // components); MFMA (j, q) then accumulates G[4j + n%4][4(n/4) + q][mu2].
  // Other K: column n = channel n, one MFMA per component.
  struct StepData {
    float a;
    float xv[K];
  };
  auto load = [&](int el, bool live) {
    StepData d;
    if constexpr (kOffsets) {
      const uint32_t o = (live ? (uint32_t)sstg[el] : 0xFFFFF000u) + (uint32_t)(((cl & 3) * K + 4 * (cl >> 2)) * 4);
      d.a = ystg[el * Cfg::YS + cl];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f4 t = buf_f4(rx, o + (uint32_t)(j * 4 * K * 4));
        d.xv[4 * j] = t[0];
        d.xv[4 * j + 1] = t[1];
        d.xv[4 * j + 2] = t[2];
        d.xv[4 * j + 3] = t[3];
      }
      return d;
    }
    const int s = sstg[el];
    const bool ok = live && s >= 0;
    d.a = live ? ystg[el * Cfg::YS + cl] : 0.0f;
    if constexpr (K == 16) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int cw = 4 * j + (cl & 3);
        const bool v = ok && cw < Cfg::CW;
        const f4 t = ld4(v ? ((size_t)s * C + c_base + cw) * K + 4 * (cl >> 2) : 0, v);
        d.xv[4 * j] = t[0];
        d.xv[4 * j + 1] = t[1];
        d.xv[4 * j + 2] = t[2];
        d.xv[4 * j + 3] = t[3];
      }
    } else {
      const bool v = ok && c_ok;
      const size_t e0 = ((size_t)(v ? s : 0) * C + c_base + (c_ok ? cl : 0)) * K;
      if constexpr (K % 4 == 0) {
#pragma unroll
        for (int q = 0; q < K / 4; ++q) {
          const f4 t = ld4(e0 + 4 * q, v);
          d.xv[4 * q] = t[0];
          d.xv[4 * q + 1] = t[1];
          d.xv[4 * q + 2] = t[2];
          d.xv[4 * q + 3] = t[3];
        }
      } else {
#pragma unroll
        for (int k = 0; k < K; ++k) d.xv[k] = ld1(e0 + k, v);
      }
    }
    return d;
  };
  auto compute = [&](const StepData& d) {
#pragma unroll
    for (int k = 0; k < K; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x4f32(d.a, d.xv[k], acc[k], 0, 0, 0);
  };

  auto task_end = [&](int row, int blk) {
    // G[c][mu1][mu2] -> LDS (over the staging area), one 16-byte store per
    // accumulator: lane (cl, kq) holds mu2 = 4 kq + v of
    //   K = 16: acc[4j + q] -> channel 4j + cl%4, mu1 = 4(cl/4) + q (row grow(mu1));
    //   else:   acc[k]      -> channel cl, mu1 = k.
    if constexpr (K == 16) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int cw = 4 * j + (cl & 3);
        if (cw < Cfg::CW) {
          float* gc = lds + cw * Cfg::GS;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<f4*>(gc + Cfg::grow(4 * (cl >> 2) + q) * K + 4 * (lane >> 4)) = acc[4 * j + q];
        }
      }
    } else if (c_ok) {
      float* gc = lds + cl * Cfg::GS;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        if constexpr (K % 4 == 0) {
          *reinterpret_cast<f4*>(gc + k * K + 4 * (lane >> 4)) = acc[k];
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int mu2 = 4 * (lane >> 4) + v;
            if (mu2 < K) gc[k * K + mu2] = acc[k][v];
          }
        }
      }
    }
#pragma unroll
    for (int k = 0; k < K; ++k) acc[k] = f4{0.f, 0.f, 0.f, 0.f};
    wave_lds_sync();
    // coupling for channel c = blk*CW + lane (lanes < CW), all output components
    if (lane < Cfg::CW) {
      const int c = blk * Cfg::CW + lane;
      const float* gc = lds + lane * Cfg::GS;
      float wr[T::P];
#pragma unroll
      for (int p = 0; p < T::P; ++p) wr[p] = w[p * C + c];
      float ov[K];
#pragma unroll
      for (int k = 0; k < K; ++k) ov[k] = 0.0f;
      float xs[TR ? K : 1];  // x[row, c, :] for grad_w
      if constexpr (TR) {
        const size_t xo = ((size_t)row * C + c) * K;
        if (xn != nullptr) {
          if constexpr (K % 4 == 0) {
#pragma unroll
            for (int q = 0; q < K / 4; ++q) {
              const f4 v = *reinterpret_cast<const f4*>(xn + xo + 4 * q);
              xs[4 * q] = v[0];
              xs[4 * q + 1] = v[1];
              xs[4 * q + 2] = v[2];
              xs[4 * q + 3] = v[3];
            }
          } else {
#pragma unroll
            for (int k = 0; k < K; ++k) xs[k] = xn[xo + k];
          }
        } else {
#pragma unroll
          for (int k = 0; k < K; ++k) xs[k] = 0.0f;
        }
      }
      float t = 0.0f;
      static_for<0, T::NT>([&](auto ii) {
        constexpr int i = decltype(ii)::value;
        constexpr eqtp_gen::CgTerm tm = T::by_out[i];
        constexpr bool first = (i == 0) || T::by_out[i - 1].p != tm.p || T::by_out[i - 1].mu3 != tm.mu3;
        constexpr bool last = (i + 1 == T::NT) || T::by_out[i + 1].p != tm.p || T::by_out[i + 1].mu3 != tm.mu3;
        const float g = gc[Cfg::grow(tm.mu1) * K + tm.mu2];
        t = first ? tm.c * g : fmaf(tm.c, g, t);
        if constexpr (last) {
          ov[tm.mu3] = fmaf(wr[tm.p], t, ov[tm.mu3]);
          if constexpr (TR) gwl[tm.p * 16 + lane] = fmaf(xs[tm.mu3], t, gwl[tm.p * 16 + lane]);
        }
      });
      if (TR && out == nullptr) return;
      float* op = out + ((size_t)row * C + c) * K;
      if constexpr (K % 4 == 0) {
#pragma unroll
        for (int q = 0; q < K / 4; ++q)
          reinterpret_cast<f4*>(op)[q] = f4{ov[4 * q], ov[4 * q + 1], ov[4 * q + 2], ov[4 * q + 3]};
      } else {
#pragma unroll
        for (int k = 0; k < K; ++k) op[k] = ov[k];
      }
    }
  };

  // load() needs the channel block of the current task: advance it after each task
  node_tasks<Cfg::PF, Cfg::NBLK, BUF>(
      N, E, row_ptr, vec, src, stage, load, compute,
      [&](int row, int blk) {
        task_end(row, blk);
        // next task's block (tasks advance by gridDim.x)
        const long long tn = (long long)row * Cfg::NBLK + blk + gridDim.x;
        c_base = (int)(tn % Cfg::NBLK) * Cfg::CW;
      });
  if constexpr (TR) {
    // the grid is a multiple of NBLK (node_grid), so every task of this wave
    // had channel block blockIdx.x % NBLK
    if (gw != nullptr && lane < Cfg::CW && (long long)blockIdx.x < (long long)N * Cfg::NBLK) {
      const int c = (int)(blockIdx.x % Cfg::NBLK) * Cfg::CW + lane;
#pragma unroll
      for (int p = 0; p < T::P; ++p) unsafeAtomicAdd(gw + p * C + c, gwl[p * 16 + lane]);
    }
  }
}
// Test-only twin: the same launch shape and node_tasks schedule, counting
// edges and summing source indices per row instead of the product (channel
// block 0 of each row reports).
template <int L, int C>
__global__ __launch_bounds__(64) void probe_node_kernel(int N, int E, const int* __restrict__ row_ptr,
                                                        const float* __restrict__ vec, const int* __restrict__ src,
                                                        int* __restrict__ count, long long* __restrict__ src_sum) {
  using Cfg = NodeCfg<L, C>;
  __shared__ __attribute__((aligned(16))) float lds[Cfg::LDS];
  const int lane = threadIdx.x & 63;
  float* ystg = lds;
  int* sstg = reinterpret_cast<int*>(lds + 64 * Cfg::YS);
  int cnt_acc = 0;
  long long sum_acc = 0;
  auto stage = [&](bool valid, float, float, float, int s) {
    ystg[lane * Cfg::YS] = valid ? 1.0f : 0.0f;  // the "harmonic" flags real slots
    sstg[lane] = s;
  };
  struct StepData {
    bool real;
    int s;
  };
  auto load = [&](int el, bool live) { return StepData{live && ystg[el * Cfg::YS] != 0.0f, sstg[el]}; };
  auto compute = [&](const StepData& d) {
    if ((lane & 15) == 0 && d.real) {
      cnt_acc += 1;
      sum_acc += d.s;
    }
  };
  auto task_end = [&](int row, int blk) {
    // lanes 0, 16, 32, 48 hold partial results; fold them
    for (int off = 16; off < 64; off <<= 1) {
      cnt_acc += __shfl_xor(cnt_acc, off);
      sum_acc += __shfl_xor(sum_acc, off);
    }
    if (blk == 0 && lane == 0) {
      count[row] = cnt_acc;
      src_sum[row] = sum_acc;
    }
    cnt_acc = 0;
    sum_acc = 0;
  };
  node_tasks<Cfg::PF, Cfg::NBLK, true>(N, E, row_ptr, vec, src, stage, load, compute, task_end);
}

// compute units of the current device, queried once per device (launches are
// on the host's hot path for small graphs); racing first queries store the
// same value
int num_cus() {
  static std::atomic<int> cached[64];
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < 64 && (n = cached[dev].load(std::memory_order_relaxed)) > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
  if (dev >= 0 && dev < 64) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

// persistent single-wave workgroups: two per SIMD.  The grid is a multiple
// of NBLK (tasks is, and so is the cap), so a wave keeps one channel block.
template <int L, int C>
static unsigned node_grid(int64_t N) {
  constexpr int NB = NodeCfg<L, C>::NBLK;
  const int64_t tasks = N * NB;
  const int64_t g = (int64_t)num_cus() * 8 / NB * NB;
  return (unsigned)(tasks < g ? tasks : g);
}

template <int L, int PS, int C>
static hipError_t launch_node(const ConvArgs& a) {
  using Cfg = NodeCfg<L, C>;
  if (a.N == 0) return hipSuccess;
  const uint64_t xs = a.x_bf16 ? 2u : 4u;
  const bool buf = (uint64_t)a.N * C * Cfg::K * xs <= kMaxBufferBytes && (uint64_t)a.E * 12u <= kMaxBufferBytes;
  const dim3 grid(node_grid<L, C>(a.N)), block(Cfg::THREADS);
  if (a.x_bf16) {
    if (buf)
      hipLaunchKernelGGL((conv_node_kernel<L, PS, C, true, true, false>), grid, block, 0, a.stream, (int)a.N,
                         (int)a.E, a.row_ptr, a.vec, a.src, a.x, a.w, a.out, nullptr, nullptr);
    else
      hipLaunchKernelGGL((conv_node_kernel<L, PS, C, false, true, false>), grid, block, 0, a.stream, (int)a.N,
                         (int)a.E, a.row_ptr, a.vec, a.src, a.x, a.w, a.out, nullptr, nullptr);
  } else {
    if (buf)
      hipLaunchKernelGGL((conv_node_kernel<L, PS, C, true, false, false>), grid, block, 0, a.stream, (int)a.N,
                         (int)a.E, a.row_ptr, a.vec, a.src, a.x, a.w, a.out, nullptr, nullptr);
    else
      hipLaunchKernelGGL((conv_node_kernel<L, PS, C, false, false, false>), grid, block, 0, a.stream, (int)a.N,
                         (int)a.E, a.row_ptr, a.vec, a.src, a.x, a.w, a.out, nullptr, nullptr);
  }
  return hipGetLastError();
}

template <int L, int PS, int C>
static hipError_t launch_node_adjoint(const BwdArgs& a) {
  using Cfg = NodeCfg<L, C>;
  hipError_t err;
  if (a.gw && (err = launch_fill_zero(a.gw, (int64_t)Tables<L, PS>::P * C, a.stream)) != hipSuccess) return err;
  if (a.N == 0) return hipSuccess;
  const bool buf = (uint64_t)a.N * C * Cfg::K * 4u <= kMaxBufferBytes && (uint64_t)a.E * 12u <= kMaxBufferBytes;
  const dim3 grid(node_grid<L, C>(a.N)), block(Cfg::THREADS);
  if (buf)
    hipLaunchKernelGGL((conv_node_kernel<L, PS, C, true, false, true>), grid, block, 0, a.stream, (int)a.N, (int)a.E,
                       a.row_ptr, a.vec, a.dst, a.gout, a.w, a.gx, a.x, a.gw);
  else
    hipLaunchKernelGGL((conv_node_kernel<L, PS, C, false, false, true>), grid, block, 0, a.stream, (int)a.N,
                       (int)a.E, a.row_ptr, a.vec, a.dst, a.gout, a.w, a.gx, a.x, a.gw);
  return hipGetLastError();
}

template <int L, int C>
static hipError_t launch_probe_node(const ProbeArgs& a) {
  using Cfg = NodeCfg<L, C>;
  if (a.N == 0) return hipSuccess;
  hipLaunchKernelGGL((probe_node_kernel<L, C>), dim3(node_grid<L, C>(a.N)), dim3(Cfg::THREADS), 0, a.stream,
                     (int)a.N, (int)a.E, a.row_ptr, (const float*)nullptr, a.src, a.count, a.src_sum);
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

template <int L, int PS>
static hipError_t dispatch_adjoint_c(const BwdArgs& a) {
  EQTP_C_SWITCH(a.C, return (launch_node_adjoint<L, PS, CC>(a)))
}

hipError_t launch_conv_backward_by_source(const BwdArgs& a) {
  switch (a.lmax * 2 + a.path_set) {
    case 0: return dispatch_adjoint_c<0, 0>(a);
    case 1: return dispatch_adjoint_c<0, 1>(a);
    case 2: return dispatch_adjoint_c<1, 0>(a);
    case 3: return dispatch_adjoint_c<1, 1>(a);
    case 4: return dispatch_adjoint_c<2, 0>(a);
    case 5: return dispatch_adjoint_c<2, 1>(a);
    case 6: return dispatch_adjoint_c<3, 0>(a);
    case 7: return dispatch_adjoint_c<3, 1>(a);
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
