// so2_device.hpp -- device pieces of the edge-aligned (SO(2)) form shared by
// the forward kernels (conv_so2.hip) and the gradients (conv_bwd_so2.hip,
// conv_bwd.hip): the sparse coupling tables, the constant rotation J and the
// pair rotations Z, the edge frame, and the rotation generators.  With R_e taking the edge
// direction to the z axis, D(R_e) = J^T Z(-theta) J Z(-phi) and
// D(R_e)^T = Z(phi) J^T Z(theta) J (E2Former-V2 page, section 2.1, and
// conv_so2.hip).
#pragma once

#include <type_traits>

#include "eqtp_device.hpp"
#include "generated/so2_tables.inc"

namespace eqtp {

template <int L, int PS>
struct So2Tables;

#define EQTP_SO2(L_, PS_, TAG)                                                     \
  template <>                                                                      \
  struct So2Tables<L_, PS_> {                                                      \
    static constexpr int P = eqtp_gen::kSo2NumPaths_##TAG;                         \
    static constexpr int NT = eqtp_gen::kSo2NumTerms_##TAG;                        \
    static constexpr const eqtp_gen::So2Term* terms = eqtp_gen::kSo2Terms_##TAG;   \
  };
EQTP_SO2(0, 0, L0_parity)
EQTP_SO2(1, 0, L1_parity)
EQTP_SO2(2, 0, L2_parity)
EQTP_SO2(3, 0, L3_parity)
EQTP_SO2(4, 0, L4_parity)
EQTP_SO2(5, 0, L5_parity)
EQTP_SO2(6, 0, L6_parity)
EQTP_SO2(0, 1, L0_so3)
EQTP_SO2(1, 1, L1_so3)
EQTP_SO2(2, 1, L2_so3)
EQTP_SO2(3, 1, L3_so3)
EQTP_SO2(4, 1, L4_so3)
EQTP_SO2(5, 1, L5_so3)
EQTP_SO2(6, 1, L6_so3)
#undef EQTP_SO2

// v <- J v (T = false) or J^T v (T = true) on the first K components
template <int K, bool T>
__device__ __forceinline__ void apply_j(float (&v)[K]) {
  constexpr int NE = T ? eqtp_gen::kJTRowStart[K] : eqtp_gen::kJRowStart[K];
  float o[K];
  static_for<0, NE>([&](auto ii) {
    constexpr int i = decltype(ii)::value;
    constexpr eqtp_gen::JEntry je = T ? eqtp_gen::kJT[i] : eqtp_gen::kJ[i];
    constexpr bool first = i == 0 || (T ? eqtp_gen::kJT[i - 1].row : eqtp_gen::kJ[i - 1].row) != je.row;
    o[je.row] = first ? je.v * v[je.col] : fmaf(je.v, v[je.col], o[je.row]);
  });
#pragma unroll
  for (int k = 0; k < K; ++k) v[k] = o[k];
}

// v <- Z(a) v: each (m cos, m sin) pair of degree l <= L rotated by m a, with
// cm[m] = cos(m a), sm[m] = sgn * sin(m a)
template <int L, int K>
__device__ __forceinline__ void apply_z(float (&v)[K], const float (&cm)[L + 1], const float (&sm)[L + 1],
                                        float sgn) {
#pragma unroll
  for (int l = 1; l <= L; ++l)
#pragma unroll
    for (int m = 1; m <= l; ++m) {
      const int c = l * l + 2 * m - 1, s = c + 1;
      const float sn = sgn * sm[m];
      const float vc = v[c], vs = v[s];
      v[c] = fmaf(cm[m], vc, -sn * vs);
      v[s] = fmaf(sn, vc, cm[m] * vs);
    }
}

// cos(m a), sin(m a) for m = 0..L from cos a, sin a
template <int L>
__device__ __forceinline__ void angle_powers(float c1, float s1, float (&cm)[L + 1], float (&sm)[L + 1]) {
  cm[0] = 1.0f;
  sm[0] = 0.0f;
#pragma unroll
  for (int m = 1; m <= L; ++m) {
    cm[m] = fmaf(cm[m - 1], c1, -sm[m - 1] * s1);
    sm[m] = fmaf(sm[m - 1], c1, cm[m - 1] * s1);
  }
}

// The edge frame of one edge vector: cos/sin of m phi and m theta for the
// pair rotations (identity for a zero vector or along the z axis, where phi is
// free), and keep = 0 for a zero vector (paths with l2 > 0 vanish there).
template <int L>
struct So2Frame {
  float cp[L + 1], sp[L + 1], ct[L + 1], st[L + 1];
  float keep;
  __device__ __forceinline__ So2Frame(float vx, float vy, float vz) {
    const float r2 = vx * vx + vy * vy + vz * vz;
    const bool nz = r2 > 0.0f;
    const float inv_r = nz ? rsqrtf(r2) : 0.0f;
    const float ux = vx * inv_r, uy = vy * inv_r, uz = nz ? vz * inv_r : 1.0f;
    const float rho2 = ux * ux + uy * uy;
    const bool tilt = rho2 > 0.0f;
    const float inv_rho = tilt ? rsqrtf(rho2) : 0.0f;
    angle_powers<L>(tilt ? ux * inv_rho : 1.0f, tilt ? uy * inv_rho : 0.0f, cp, sp);
    angle_powers<L>(uz, tilt ? rho2 * inv_rho : 0.0f, ct, st);
    keep = nz ? 1.0f : 0.0f;
  }
  So2Frame() = default;
  // LDS record of FS floats (16-byte aligned): cp, sp, ct, st, keep, and one
  // spare word (SRC) for the caller
  static constexpr int SRC = 4 * (L + 1) + 1;
  static constexpr int FS = (SRC + 1 + 3) / 4 * 4;
  __device__ __forceinline__ void store(float* __restrict__ f) const {
#pragma unroll
    for (int m = 0; m <= L; ++m) {
      f[m] = cp[m];
      f[L + 1 + m] = sp[m];
      f[2 * (L + 1) + m] = ct[m];
      f[3 * (L + 1) + m] = st[m];
    }
    f[4 * (L + 1)] = keep;
  }
  __device__ __forceinline__ void load(const float* __restrict__ f) {
#pragma unroll
    for (int m = 0; m <= L; ++m) {
      cp[m] = f[m];
      sp[m] = f[L + 1 + m];
      ct[m] = f[2 * (L + 1) + m];
      st[m] = f[3 * (L + 1) + m];
    }
    keep = f[4 * (L + 1)];
  }
};

// v <- D(R_e) v (into the edge frame) and v <- D(R_e)^T v (back)
template <int L, int K>
__device__ __forceinline__ void so2_rotate_in(float (&v)[K], const So2Frame<L>& f) {
  apply_z<L>(v, f.cp, f.sp, -1.0f);
  apply_j<K, false>(v);
  apply_z<L>(v, f.ct, f.st, -1.0f);
  apply_j<K, true>(v);
}
template <int L, int K>
__device__ __forceinline__ void so2_rotate_out(float (&v)[K], const So2Frame<L>& f) {
  apply_j<K, false>(v);
  apply_z<L>(v, f.ct, f.st, 1.0f);
  apply_j<K, true>(v);
  apply_z<L>(v, f.cp, f.sp, 1.0f);
}

// sum_r a[r] (L v)[r] for the generator of rotations L = L_x (LX) or L_y
// (L_a = d/de D(R_a(e)) at e = 0), rows of the table walked with the entries
// as instruction immediates.  With x', g' the features in the edge frame,
// u' = P_w x' and v' = P_w^T g', the loss's tangential derivatives at the
// frame's pole are G_x = -(v' . L_y x' + u' . L_y g') and
// G_y = v' . L_x x' + u' . L_x g' (the coupling's invariance moves the
// derivative of the harmonics onto x' and g'; conv_bwd_so2.hip)
template <int K, bool LX>
__device__ __forceinline__ float gen_form(const float (&a)[K], const float (&v)[K]) {
  constexpr int NE = LX ? eqtp_gen::kLxRowStart[K] : eqtp_gen::kLyRowStart[K];
  float acc = 0.0f, t = 0.0f;
  static_for<0, NE>([&](auto ii) {
    constexpr int i = decltype(ii)::value;
    constexpr eqtp_gen::JEntry je = LX ? eqtp_gen::kLx[i] : eqtp_gen::kLy[i];
    constexpr bool first = i == 0 || (LX ? eqtp_gen::kLx[i - 1].row : eqtp_gen::kLy[i - 1].row) != je.row;
    constexpr bool last = i + 1 == NE || (LX ? eqtp_gen::kLx[i + 1].row : eqtp_gen::kLy[i + 1].row) != je.row;
    t = first ? je.v * v[je.col] : fmaf(je.v, v[je.col], t);
    if constexpr (last) acc = fmaf(a[je.row], t, acc);
  });
  return acc;
}

// dL/dvec = R_e^T (G_x, G_y, 0) / |vec| for the edge frame f (R_e = R_y(-theta) R_z(-phi))
template <int L>
__device__ __forceinline__ void frame_gradient(const So2Frame<L>& f, float gxe, float gye, float inv_r, float& g0,
                                               float& g1, float& g2) {
  if constexpr (L >= 1) {
    const float a = gxe * inv_r, b = gye * inv_r;
    g0 = fmaf(a * f.ct[1], f.cp[1], -b * f.sp[1]);
    g1 = fmaf(a * f.ct[1], f.sp[1], b * f.cp[1]);
    g2 = -a * f.st[1];
  } else {
    g0 = g1 = g2 = 0.0f;
  }
}

}  // namespace eqtp
