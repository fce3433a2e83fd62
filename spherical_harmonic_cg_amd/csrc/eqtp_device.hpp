// eqtp_device.hpp -- device-side building blocks shared by the gfx950 kernels:
// real spherical harmonics, the radial basis, compile-time coupling tables and
// small wave-level helpers.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <utility>

#include "generated/cg_tables.inc"

namespace eqtp {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

__host__ __device__ constexpr int num_comp(int L) { return (L + 1) * (L + 1); }

// ---------------------------------------------------------------------------
// Compile-time coupling tables (generated from the Racah formula, see
// gen_cg_table.py).  Tables<L, PS>::by_out lists the non-zero real-basis
// coefficients sorted by (mu3, p, mu1, mu2); by_path by (p, mu3, mu1, mu2).
// ---------------------------------------------------------------------------
template <int L, int PS>
struct Tables;

#define EQTP_TABLES(L_, PS_, TAG)                                                     \
  template <>                                                                         \
  struct Tables<L_, PS_> {                                                            \
    static constexpr int P = eqtp_gen::kNumPaths_##TAG;                               \
    static constexpr int NT = eqtp_gen::kNumTerms_##TAG;                              \
    static constexpr const eqtp_gen::CgTerm* by_out = eqtp_gen::kTermsByOut_##TAG;    \
    static constexpr const eqtp_gen::CgTerm* by_path = eqtp_gen::kTermsByPath_##TAG;  \
    static constexpr const eqtp_gen::PathLs* paths = eqtp_gen::kPaths_##TAG;          \
  };
EQTP_TABLES(0, 0, L0_parity)
EQTP_TABLES(1, 0, L1_parity)
EQTP_TABLES(2, 0, L2_parity)
EQTP_TABLES(3, 0, L3_parity)
EQTP_TABLES(0, 1, L0_so3)
EQTP_TABLES(1, 1, L1_so3)
EQTP_TABLES(2, 1, L2_so3)
EQTP_TABLES(3, 1, L3_so3)
#undef EQTP_TABLES

// Calls f(std::integral_constant<int, B + i>) for i = 0 .. E-B-1, fully
// expanded at compile time so that every table lookup inside f folds into an
// instruction immediate.
template <int B, class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, B + I>{}), ...);
}
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (E > B) static_for_impl<B>(static_cast<F&&>(f), std::make_integer_sequence<int, E - B>{});
}

// ---------------------------------------------------------------------------
// Real spherical harmonics for l <= L of an (unnormalised) edge vector,
// components in the page order (l0, l1c, l1s, l2c, l2s, ...).  The vector is
// normalised with one reciprocal square root, as the Batmobile page does
// (section "2. register intermediate computation").  A zero vector gives
// (Y00, 0, ..., 0).  Y[k] for k >= (L+1)^2 is set to 0.
// ---------------------------------------------------------------------------
template <int L>
__device__ __forceinline__ void sh_eval(float vx, float vy, float vz, float (&Y)[16]) {
  using namespace eqtp_gen;
  const float r2 = vx * vx + vy * vy + vz * vz;
  const bool nz = r2 > 0.0f;
  const float inv = nz ? rsqrtf(r2) : 0.0f;
  const float x = vx * inv, y = vy * inv, z = vz * inv;
  const float m = nz ? 1.0f : 0.0f;  // zero vector: every l > 0 component is 0
#pragma unroll
  for (int k = 0; k < 16; ++k) Y[k] = 0.0f;
  Y[0] = kShY00;
  if constexpr (L >= 1) {
    Y[1] = kShC1 * z;
    Y[2] = -kShC1 * x;
    Y[3] = -kShC1 * y;
  }
  if constexpr (L >= 2) {
    const float zz = z * z, xx = x * x, yy = y * y;
    Y[4] = m * kShC20 * (3.0f * zz - 1.0f);
    Y[5] = -kShC21 * x * z;
    Y[6] = -kShC21 * y * z;
    Y[7] = kShC22 * (xx - yy);
    Y[8] = 2.0f * kShC22 * x * y;
    if constexpr (L >= 3) {
      const float f = 5.0f * zz - 1.0f;
      Y[9] = m * kShC30 * z * (5.0f * zz - 3.0f);
      Y[10] = -kShC31 * x * f;
      Y[11] = -kShC31 * y * f;
      Y[12] = kShC32 * z * (xx - yy);
      Y[13] = 2.0f * kShC32 * x * y * z;
      Y[14] = -kShC33 * x * (xx - 3.0f * yy);
      Y[15] = -kShC33 * y * (3.0f * xx - yy);
    }
  }
}

// ---------------------------------------------------------------------------
// Radial basis: R_n(r) = sin(n pi r / r_c) / r * u(r / r_c), n = 1..NB, with
// the p = 6 polynomial envelope u(d) = 1 - 28 d^6 + 48 d^7 - 21 d^8 (d < 1,
// else 0) and the limit n pi / r_c at r = 0.  sin(n t) by the Chebyshev
// recurrence sin((n+1)t) = 2 cos t sin(nt) - sin((n-1)t).
// ---------------------------------------------------------------------------
template <int NB>
__device__ __forceinline__ void radial_basis(float r, float inv_rc, float (&R)[NB]) {
  const float d = r * inv_rc;
  if (!(d < 1.0f)) {
#pragma unroll
    for (int n = 0; n < NB; ++n) R[n] = 0.0f;
    return;
  }
  const float d2 = d * d, d6 = d2 * d2 * d2;
  const float env = 1.0f + d6 * (-28.0f + d * (48.0f - 21.0f * d));
  if (r == 0.0f) {
#pragma unroll
    for (int n = 0; n < NB; ++n) R[n] = (float)(n + 1) * eqtp_gen::kPiF * inv_rc;
    return;
  }
  float s1, c1;
  sincosf(eqtp_gen::kPiF * d, &s1, &c1);
  const float scale = env / r;
  float sm1 = 0.0f, s = s1;
  const float c2 = 2.0f * c1;
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    R[n] = s * scale;
    const float sn = c2 * s - sm1;
    sm1 = s;
    s = sn;
  }
}

// Clamp an index read from memory into [0, n-1] (memory safety for arbitrary
// index contents; n >= 1).
__device__ __forceinline__ int clamp_index(int v, int n) { return v < 0 ? 0 : (v >= n ? n - 1 : v); }

// LDS visibility inside one wavefront: LDS operations of a wave complete in
// issue order; this stops the compiler from moving them across the point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// Raw buffer loads.  A load whose byte offset falls outside the resource
// returns zeros without touching memory, so masked loads need no branch and
// the compiler can count outstanding loads statically (which a branch around
// each load prevents).  Resources cover < 4 GiB; callers check the size.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutOfRange = 0xFFFFFFF0u;   // any offset at or past the end reads as zero
constexpr uint64_t kMaxBufferBytes = 0xFFFF0000ull;

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint64_t bytes) {
  // word 3 of a gfx9 buffer resource: 32-bit data format, no swizzle
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)(uint32_t)bytes, 0x00020000);
}
__device__ __forceinline__ f4 buf_f4(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ float buf_f32(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
__device__ __forceinline__ int buf_i32(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(int, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

// Round-to-nearest-even float -> bfloat16.
__device__ __forceinline__ __bf16 to_bf16(float f) { return (__bf16)f; }

}  // namespace eqtp
