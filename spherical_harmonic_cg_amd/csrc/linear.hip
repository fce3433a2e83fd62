// linear.hip -- per-l channel linear out[n,c',l m] = sum_c W[l,c',c] h[n,c,l m]
// on the matrix cores (the one dense contraction of the path).
//
// A workgroup (4 waves) takes 16 consecutive nodes -- one contiguous
// 16*C*K-element block of h, fp32 or bf16 in memory.  It stages, in the
// operand type (bf16 or fp32):
//   * W as [l][c'][c] with rows padded so that the 16-byte operand reads of
//     16 consecutive rows fall in distinct LDS banks (when it fits in LDS;
//     otherwise the A operands are read from global memory, L2-resident);
//   * the h tile transposed to [m][node][c] (two channels per thread, plane
//     stride padded to spread the m-planes of a store over banks).
// Work units are (4 consecutive components m, 16 output channels); for each,
// the 16x16 tiles D[c'][node] come from v_mfma_f32_16x16x32_bf16 (bf16
// products: operands held as bf16 in memory, or fp32 rounded to nearest-even
// bf16 when staged; fp32 accumulation) or v_mfma_f32_16x16x4_f32 (fp32 mode).
// Lane (i, k) holds D[c'0+4k+v][node i] for the four m of the unit, i.e.
// out[node i][c'][m..m+3].  When every wave is done, the (dead) input staging
// is reused as the fp32 output tile in the global layout and the tile leaves
// with coalesced 16-byte stores.  Bytes per node: C K (h once, 4 or 2 bytes
// each) + 4 C K (out once); flops 2 C^2 K: bound by HBM bandwidth.
#include <type_traits>

#include "eqtp_device.hpp"
#include "eqtp_kernels.hpp"

namespace eqtp {

template <bool BF16>
struct LinOp;
template <>
struct LinOp<true> {
  typedef __bf16 T;
  static constexpr int KSTEP = 32;  // input channels per MFMA
  static constexpr int PAD = 8;     // row padding (elements): 16 bytes
};
template <>
struct LinOp<false> {
  typedef float T;
  static constexpr int KSTEP = 16;  // four 16x16x4 MFMAs per 16 input channels
  static constexpr int PAD = 4;
};

template <int L, int C, bool BF16>
struct LinCfg {
  using Op = LinOp<BF16>;
  typedef typename Op::T T;
  static constexpr int K = num_comp(L);
  static constexpr int TN = 16;                      // nodes per workgroup (MFMA columns)
  static constexpr int RS = C + Op::PAD;             // LDS row stride (elements)
  static constexpr int ES = (int)sizeof(T);
  // m-plane stride in 4-byte words: TN rows plus 4 words (keeps 16-byte alignment; planes 4 apart land
  // 16 banks apart)
  static constexpr int PLANE_W = (TN * RS * ES) / 4 + 4;
  static constexpr int PLANE = PLANE_W * 4 / ES;     // in elements
  static constexpr int H_ELEMS = K * PLANE;
  static constexpr int W_ELEMS = (L + 1) * C * RS;
  static constexpr int LDS_BYTES_FULL = (H_ELEMS + W_ELEMS) * ES;
  static constexpr bool W_LDS = LDS_BYTES_FULL <= 160 * 1024;
  static constexpr int NS = C * K + 4;              // output tile node stride (floats)
  static constexpr int OUT_FLOATS = TN * NS;
  static constexpr int LDS_ELEMS_IN = H_ELEMS + (W_LDS ? W_ELEMS : 0);
  static constexpr int LDS_BYTES = LDS_ELEMS_IN * ES > OUT_FLOATS * 4 ? LDS_ELEMS_IN * ES : OUT_FLOATS * 4;
  static constexpr int CT = (C + 15) / 16;           // 16-row output channel tiles
  static constexpr int MQ = (K + 3) / 4;             // component quads
  static constexpr int UNITS = MQ * CT;
  static constexpr int WAVES = 4;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  static_assert(C % 8 == 0, "channels must be a multiple of 8");
};

// 4 consecutive stored elements widened to fp32 (one 16-byte or 8-byte load; a bf16 value is the upper
// half of the fp32 with the same bits)
__device__ __forceinline__ f4 ld4s(const float* p) { return *reinterpret_cast<const f4*>(p); }
__device__ __forceinline__ f4 ld4s(const __bf16* p) {
  const uint2 t = *reinterpret_cast<const uint2*>(p);
  return f4{__uint_as_float(t.x << 16), __uint_as_float(t.x & 0xffff0000u), __uint_as_float(t.y << 16),
            __uint_as_float(t.y & 0xffff0000u)};
}

__device__ __forceinline__ int l_of(int m) { return m >= 9 ? 3 : (m >= 4 ? 2 : (m >= 1 ? 1 : 0)); }

template <class T>
__device__ __forceinline__ T to_op(float f);
template <>
__device__ __forceinline__ __bf16 to_op<__bf16>(float f) { return to_bf16(f); }
template <>
__device__ __forceinline__ float to_op<float>(float f) { return f; }

// S: the element type of h and W in memory (float or __bf16)
template <int L, int C, bool BF16, class S>
__global__ __launch_bounds__(256) void linear_kernel(int N, const S* __restrict__ h, const S* __restrict__ W,
                                                     float* __restrict__ out) {
  using Cfg = LinCfg<L, C, BF16>;
  using Op = typename Cfg::Op;
  typedef typename Cfg::T T;
  constexpr int K = Cfg::K;
  constexpr int TN = Cfg::TN;
  constexpr int RS = Cfg::RS;
  __shared__ __attribute__((aligned(16))) unsigned char lds_raw[Cfg::LDS_BYTES];
  T* hT = reinterpret_cast<T*>(lds_raw);   // [K][PLANE]: plane m holds rows node*RS + c
  T* Wl = hT + Cfg::H_ELEMS;               // [L+1][C][RS]
  float* otile = reinterpret_cast<float*>(lds_raw);  // after the products: [node][NS] output tile
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int n0 = blockIdx.x * TN;
  const int nv = min(TN, N - n0);
  const size_t base = (size_t)n0 * C * K;

  // 1. stage W (once per workgroup) and the h tile: every global load is
  //    issued before the first LDS store so their latencies overlap.
  constexpr int WF4 = Cfg::W_LDS ? (L + 1) * C * C / 4 : 0;
  constexpr int W_IT = (WF4 + 255) / 256;
  // bf16 in memory and in LDS, K a multiple of 8: units of (node, channel pair, 8 components), one
  // 16-byte load per channel, the bits stored as they are (two channels per 4-byte LDS store)
  constexpr bool OCT = std::is_same<S, __bf16>::value && BF16 && K % 8 == 0;
  constexpr int HU8 = OCT ? TN * (C / 2) * (K / 8) : 0;
  constexpr int H8_IT = (HU8 + 255) / 256;
  constexpr int HU = (!OCT && K % 4 == 0) ? TN * (C / 2) * (K / 4) : 0;  // (node, channel pair, m quad) units
  constexpr int H_IT = (HU + 255) / 256;
  f4 wbuf[W_IT > 0 ? W_IT : 1];
  f4 ha[H_IT > 0 ? H_IT : 1], hb[H_IT > 0 ? H_IT : 1];
  uint4 h8a[H8_IT > 0 ? H8_IT : 1], h8b[H8_IT > 0 ? H8_IT : 1];
#pragma unroll
  for (int it = 0; it < W_IT; ++it) {
    const int i = tid + it * 256;
    wbuf[it] = i < WF4 ? ld4s(W + 4 * i) : f4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int it = 0; it < H_IT; ++it) {
    const int u = tid + it * 256;
    const int mq = u % (K / 4 > 0 ? K / 4 : 1);
    const int cp = (u / (K / 4 > 0 ? K / 4 : 1)) % (C / 2);
    const int n = u / ((K / 4 > 0 ? K / 4 : 1) * (C / 2));
    ha[it] = hb[it] = f4{0.f, 0.f, 0.f, 0.f};
    if (u < HU && n < nv) {
      const S* src = h + base + ((size_t)n * C + 2 * cp) * K + 4 * mq;
      ha[it] = ld4s(src);
      hb[it] = ld4s(src + K);
    }
  }
  if constexpr (OCT) {
#pragma unroll
    for (int it = 0; it < H8_IT; ++it) {
      const int u = tid + it * 256;
      const int mo = u % (K / 8);
      const int cp = (u / (K / 8)) % (C / 2);
      const int n = u / ((K / 8) * (C / 2));
      h8a[it] = h8b[it] = uint4{0u, 0u, 0u, 0u};
      if (u < HU8 && n < nv) {
        const S* src = h + base + ((size_t)n * C + 2 * cp) * K + 8 * mo;
        h8a[it] = *reinterpret_cast<const uint4*>(src);
        h8b[it] = *reinterpret_cast<const uint4*>(src + K);
      }
    }
  }
#pragma unroll
  for (int it = 0; it < W_IT; ++it) {
    const int i = tid + it * 256;
    if (i < WF4) {
      const int e = 4 * i;
      const int row = e / C, c = e - row * C;  // row = l*C + c'
      T* d = Wl + row * RS + c;
#pragma unroll
      for (int j = 0; j < 4; ++j) d[j] = to_op<T>(wbuf[it][j]);
    }
  }
#pragma unroll
  for (int it = 0; it < H_IT; ++it) {
    const int u = tid + it * 256;
    if (u < HU) {
      const int mq = u % (K / 4 > 0 ? K / 4 : 1);
      const int cp = (u / (K / 4 > 0 ? K / 4 : 1)) % (C / 2);
      const int n = u / ((K / 4 > 0 ? K / 4 : 1) * (C / 2));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        T* d = hT + (4 * mq + q) * Cfg::PLANE + n * RS + 2 * cp;
        d[0] = to_op<T>(ha[it][q]);
        d[1] = to_op<T>(hb[it][q]);
      }
    }
  }
  if constexpr (OCT) {
#pragma unroll
    for (int it = 0; it < H8_IT; ++it) {
      const int u = tid + it * 256;
      if (u < HU8) {
        const int mo = u % (K / 8);
        const int cp = (u / (K / 8)) % (C / 2);
        const int n = u / ((K / 8) * (C / 2));
        const uint32_t wa[4] = {h8a[it].x, h8a[it].y, h8a[it].z, h8a[it].w};
        const uint32_t wb[4] = {h8b[it].x, h8b[it].y, h8b[it].z, h8b[it].w};
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          // component 8 mo + q of channels 2cp (low half) and 2cp + 1 (high half)
          const uint32_t a = q & 1 ? wa[q >> 1] >> 16 : wa[q >> 1] & 0xffffu;
          const uint32_t b = q & 1 ? wb[q >> 1] & 0xffff0000u : wb[q >> 1] << 16;
          *reinterpret_cast<uint32_t*>(hT + (8 * mo + q) * Cfg::PLANE + n * RS + 2 * cp) = a | b;
        }
      }
    }
  }
  if constexpr (K % 4 != 0) {
    for (int f = tid; f < TN * C * K; f += 256) {
      const int n = f / (C * K);
      const int rem = f - n * (C * K);
      const int c = rem / K;
      const int m = rem - c * K;
      hT[m * Cfg::PLANE + n * RS + c] = to_op<T>(n < nv ? (float)h[base + f] : 0.0f);
    }
  }
  __syncthreads();

  // 2. units (m quad, output tile) -> MFMA; results wait in registers
  const int i16 = lane & 15;
  const int kq = lane >> 4;
  constexpr int UPW = (Cfg::UNITS + Cfg::WAVES - 1) / Cfg::WAVES;  // units per wave
  f4 res[UPW][4];
#pragma unroll
  for (int uu = 0; uu < UPW; ++uu) {
    const int unit = wv + uu * Cfg::WAVES;
#pragma unroll
    for (int q = 0; q < 4; ++q) res[uu][q] = f4{0.f, 0.f, 0.f, 0.f};
    if (unit >= Cfg::UNITS) continue;
    const int mq = unit / Cfg::CT;
    const int ct = unit - mq * Cfg::CT;
    const int co = ct * 16 + i16;  // A row supplied by this lane
    const bool co_ok = co < C;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int m = 4 * mq + q;
      if (m >= K) continue;
      const int l = l_of(m);
      const T* hrow = hT + m * Cfg::PLANE + i16 * RS;
      f4 acc = f4{0.f, 0.f, 0.f, 0.f};
      if constexpr (BF16) {
#pragma unroll
        for (int ci0 = 0; ci0 < C; ci0 += 32) {
          const int cb = ci0 + 8 * kq;
          bf16x8 a8, b8;
          if (cb < C) {
            b8 = *reinterpret_cast<const bf16x8*>(hrow + cb);
            if constexpr (Cfg::W_LDS) {
              a8 = *reinterpret_cast<const bf16x8*>(Wl + (l * C + (co_ok ? co : 0)) * RS + cb);
            } else {
              const S* wr = W + ((size_t)l * C + (co_ok ? co : 0)) * C + cb;
              const f4 w0 = ld4s(wr), w1 = ld4s(wr + 4);
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                a8[j] = to_bf16(w0[j]);
                a8[4 + j] = to_bf16(w1[j]);
              }
            }
            if (!co_ok) {
#pragma unroll
              for (int j = 0; j < 8; ++j) a8[j] = (__bf16)0.0f;
            }
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              a8[j] = (__bf16)0.0f;
              b8[j] = (__bf16)0.0f;
            }
          }
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, b8, acc, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int ci0 = 0; ci0 < C; ci0 += 16) {
          const int cb = ci0 + 4 * kq;
          f4 a4 = f4{0.f, 0.f, 0.f, 0.f}, b4 = a4;
          if (cb < C) {
            b4 = *reinterpret_cast<const f4*>(hrow + cb);
            if (co_ok) {
              if constexpr (Cfg::W_LDS) a4 = *reinterpret_cast<const f4*>(Wl + (l * C + co) * RS + cb);
              else a4 = ld4s(W + ((size_t)l * C + co) * C + cb);
            }
          }
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[s4], b4[s4], acc, 0, 0, 0);
        }
      }
      res[uu][q] = acc;
    }
  }
  __syncthreads();  // inputs are dead: the LDS now holds the output tile

  // 3. lane (i16, kq): out[node i16][ct*16 + 4kq + v][4mq + q] = res[q][v] -> LDS tile (global layout,
  //    node stride padded by 4 words so 8 lanes' 16-byte writes hit distinct banks)
#pragma unroll
  for (int uu = 0; uu < UPW; ++uu) {
    const int unit = wv + uu * Cfg::WAVES;
    if (unit >= Cfg::UNITS) continue;
    const int mq = unit / Cfg::CT;
    const int ct = unit - mq * Cfg::CT;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int c2 = ct * 16 + 4 * kq + v;
      if (c2 >= C) continue;
      float* op = otile + i16 * Cfg::NS + c2 * K + 4 * mq;
      if constexpr (K % 4 == 0) {
        *reinterpret_cast<f4*>(op) = f4{res[uu][0][v], res[uu][1][v], res[uu][2][v], res[uu][3][v]};
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (4 * mq + q < K) op[q] = res[uu][q][v];
      }
    }
  }
  __syncthreads();

  // 4. coalesced 16-byte stores of the valid nodes
  constexpr int CK4 = C * K / 4;
  f4* ob = reinterpret_cast<f4*>(out + base);
  for (int i = tid; i < nv * CK4; i += 256) {
    const int n = i / CK4;
    const int j = i - n * CK4;
    ob[i] = *reinterpret_cast<const f4*>(otile + n * Cfg::NS + 4 * j);
  }
}

// ---------------------------------------------------------------------------
// lmax 4..6: a workgroup takes TN = 4 nodes (their K planes would not fit in
// LDS with 16 nodes).  MFMA columns are the (node, m) pairs of one degree l
// (TN (2l+1) of them, in tiles of 16), rows are 16 output channels, k runs
// over the input channels, so each tile uses the single weight matrix W[l].
// The h tile is staged transposed to rows (node, m) of C channels (operand
// type), the results go through LDS to the global layout and leave with
// coalesced stores.
// ---------------------------------------------------------------------------
template <int L, int C, bool BF16>
struct LinColsCfg {
  using Op = LinOp<BF16>;
  typedef typename Op::T T;
  static constexpr int K = num_comp(L);
  static constexpr int TN = C >= 128 ? 2 : 4;   // nodes per workgroup
  static constexpr int RS = C + Op::PAD;        // h row stride (elements): 16-byte rows
  static constexpr int H_BYTES = (TN * K * RS * (int)sizeof(T) + 15) / 16 * 16;
  static constexpr int O_BYTES = TN * C * K * 4;
  static constexpr int LDS_BYTES = H_BYTES + O_BYTES;  // input and output tiles side by side
  static constexpr int OT = (C + 15) / 16;      // output channel tiles
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <int L, int C, bool BF16, class S>
__global__ __launch_bounds__(256) void linear_cols_kernel(int N, const S* __restrict__ h, const S* __restrict__ W,
                                                          float* __restrict__ out) {
  using Cfg = LinColsCfg<L, C, BF16>;
  typedef typename Cfg::T T;
  constexpr int K = Cfg::K;
  constexpr int TN = Cfg::TN;
  constexpr int RS = Cfg::RS;
  __shared__ __attribute__((aligned(16))) unsigned char lds_raw[Cfg::LDS_BYTES];
  T* hT = reinterpret_cast<T*>(lds_raw);                              // [(node, m)][RS]
  float* otile = reinterpret_cast<float*>(lds_raw + Cfg::H_BYTES);    // [node][C][K]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int i16 = lane & 15;
  const int kq = lane >> 4;
  const int n0 = blockIdx.x * TN;
  const int nv = min(TN, N - n0);
  const size_t base = (size_t)n0 * C * K;

  // 1. stage h: element (node, c, m) -> row node*K + m, column c
  for (int f = tid; f < TN * C * K; f += 256) {
    const int node = f / (C * K);
    const int rem = f - node * (C * K);
    const int c = rem / K;
    const int m = rem - c * K;
    hT[(node * K + m) * RS + c] = to_op<T>(node < nv ? (float)h[base + f] : 0.0f);
  }
  __syncthreads();

  // 2. units (l, column tile, output tile), dealt round-robin to the waves;
  //    lane (column i16, group kq) ends with D[co = 16 ot + 4 kq + v][column]
  int unit = 0;
  for (int l = 0; l <= L; ++l) {
    const int width = 2 * l + 1;
    const int ncol = TN * width;
    const int ctn = (ncol + 15) / 16;
    for (int ct = 0; ct < ctn; ++ct) {
      for (int ot = 0; ot < Cfg::OT; ++ot, ++unit) {
        if ((unit & 3) != wv) continue;
        const int n = ct * 16 + i16;  // B column supplied by this lane
        const bool n_ok = n < ncol;
        const int node = n_ok ? n / width : 0;
        const int m = l * l + (n_ok ? n - node * width : 0);
        const T* hrow = hT + (node * K + m) * RS;
        const int co = ot * 16 + i16;  // A row supplied by this lane
        const bool co_ok = co < C;
        f4 acc = f4{0.f, 0.f, 0.f, 0.f};
        if constexpr (BF16) {
#pragma unroll
          for (int ci0 = 0; ci0 < C; ci0 += 32) {
            const int cb = ci0 + 8 * kq;
            bf16x8 a8, b8;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
              a8[j] = (__bf16)0.0f;
              b8[j] = (__bf16)0.0f;
            }
            if (cb < C) {
              if (n_ok) b8 = *reinterpret_cast<const bf16x8*>(hrow + cb);
              if (co_ok) {
                const S* wr = W + ((size_t)l * C + co) * C + cb;
                const f4 w0 = ld4s(wr), w1 = ld4s(wr + 4);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                  a8[j] = to_bf16(w0[j]);
                  a8[4 + j] = to_bf16(w1[j]);
                }
              }
            }
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, b8, acc, 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int ci0 = 0; ci0 < C; ci0 += 16) {
            const int cb = ci0 + 4 * kq;
            f4 a4 = f4{0.f, 0.f, 0.f, 0.f}, b4 = a4;
            if (cb < C) {
              if (n_ok) b4 = *reinterpret_cast<const f4*>(hrow + cb);
              if (co_ok) a4 = ld4s(W + ((size_t)l * C + co) * C + cb);
            }
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a4[s4], b4[s4], acc, 0, 0, 0);
          }
        }
        if (n_ok) {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int c2 = ot * 16 + 4 * kq + v;
            if (c2 < C) otile[(node * C + c2) * K + m] = acc[v];
          }
        }
      }
    }
  }
  __syncthreads();

  // 3. coalesced stores of the valid nodes
  constexpr int CK = C * K;
  if constexpr (CK % 4 == 0) {
    f4* ob = reinterpret_cast<f4*>(out + base);
    for (int i = tid; i < nv * CK / 4; i += 256) ob[i] = *reinterpret_cast<const f4*>(otile + 4 * i);
  } else {
    for (int i = tid; i < nv * CK; i += 256) out[base + i] = otile[i];
  }
}

template <int L, int C, bool BF16, class S>
static hipError_t launch_linear_t(int64_t N, const void* h, const void* W, float* out, hipStream_t stream) {
  const S* hs = static_cast<const S*>(h);
  const S* ws = static_cast<const S*>(W);
  if constexpr (L <= 3) {
    const unsigned blocks = (unsigned)((N + 15) / 16);
    hipLaunchKernelGGL((linear_kernel<L, C, BF16, S>), dim3(blocks), dim3(256), 0, stream, (int)N, hs, ws, out);
  } else {
    const unsigned blocks = (unsigned)((N + LinColsCfg<L, C, BF16>::TN - 1) / LinColsCfg<L, C, BF16>::TN);
    hipLaunchKernelGGL((linear_cols_kernel<L, C, BF16, S>), dim3(blocks), dim3(256), 0, stream, (int)N, hs, ws, out);
  }
  return hipGetLastError();
}

// mode 0: fp32 storage and products; 1: bf16 storage and products; 2: fp32 storage, bf16 products
template <int L, int C>
static hipError_t launch_linear_mode(int64_t N, int mode, const void* h, const void* W, float* out, hipStream_t s) {
  if (mode == 0) return launch_linear_t<L, C, false, float>(N, h, W, out, s);
  if (mode == 1) return launch_linear_t<L, C, true, __bf16>(N, h, W, out, s);
  return launch_linear_t<L, C, true, float>(N, h, W, out, s);
}

template <int L>
static hipError_t dispatch_linear_c(int64_t N, int C, int mode, const void* h, const void* W, float* out,
                                    hipStream_t s) {
  switch (C) {
    case 8: return launch_linear_mode<L, 8>(N, mode, h, W, out, s);
    case 16: return launch_linear_mode<L, 16>(N, mode, h, W, out, s);
    case 32: return launch_linear_mode<L, 32>(N, mode, h, W, out, s);
    case 64: return launch_linear_mode<L, 64>(N, mode, h, W, out, s);
    case 128: return launch_linear_mode<L, 128>(N, mode, h, W, out, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_linear(int64_t N, int C, int lmax, int mode, const void* h, const void* W, float* out,
                         hipStream_t stream) {
  if (N == 0) return hipSuccess;
  if (mode < 0 || mode > 2) return hipErrorInvalidValue;
  switch (lmax) {
    case 0: return dispatch_linear_c<0>(N, C, mode, h, W, out, stream);
    case 1: return dispatch_linear_c<1>(N, C, mode, h, W, out, stream);
    case 2: return dispatch_linear_c<2>(N, C, mode, h, W, out, stream);
    case 3: return dispatch_linear_c<3>(N, C, mode, h, W, out, stream);
    case 4: return dispatch_linear_c<4>(N, C, mode, h, W, out, stream);
    case 5: return dispatch_linear_c<5>(N, C, mode, h, W, out, stream);
    case 6: return dispatch_linear_c<6>(N, C, mode, h, W, out, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace eqtp
