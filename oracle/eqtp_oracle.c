/*
 * eqtp_oracle.c -- plain fp64 CPU oracle for the equivariant message-passing
 * convolution (spherical harmonics -> Clebsch-Gordan tensor product -> sum into
 * the destination node), the per-l channel linear and the standalone
 * spherical harmonics.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or generator with the HIP library: every constant here
 * (Legendre recursion, Racah formula, complex->real change of basis, path
 * enumeration) is computed from its textbook definition at run time.
 *
 * Everything is computed in double precision from the caller's float32
 * inputs, in the plain loop order of the definition, with no blocking, fusion
 * or reordering.  Loops over independent outputs (destination rows, nodes,
 * edges) are shared out over OpenMP threads; every output element still
 * receives its terms in the same order, so the result does not depend on the
 * thread count (checked bit for bit by the tests).
 *
 * Sources (the Batmobile page, "Batmobile CUDA kernel optimisation: a 10-20x
 * acceleration strategy for equivariant graph neural networks"):
 *   - section "equivariant GNN compute bottleneck": the core operation is real
 *     spherical harmonics of the edge direction, a Clebsch-Gordan tensor
 *     product with the source node's features, and message passing;
 *   - section "2. register intermediate computation": real SH of the unit edge
 *     vector; Y00 = 0.28209479177387814, Y10 = 0.4886025119029199*nz,
 *     Y11c = -0.4886025119029199*nx, Y11s = -0.4886025119029199*ny, in that
 *     declaration order (which fixes the Condon-Shortley phase and the
 *     per-l component order l0, l1c, l1s, l2c, l2s, ...); higher orders "are
 *     handled the same way";
 *   - section "1. compile-time constants": Clebsch-Gordan coefficients indexed
 *     by a path index (34 entries, i.e. every (l1,l2,l3<=3) triangle triple);
 *   - section "3. operator fusion": edge vectors [E,3], node features
 *     [N,C,16], source indices [E]; one message per edge.
 * The gradients (fixed and radial weights) are those of L = sum gout * out,
 * written out term by term from the forward's definition; the radial ones
 * add the derivative of the radial basis (product and chain rule).
 * Readings where the page is silent (all stated in the design notes):
 *   path weights are per path and per channel (channel-wise "uvu" product),
 *   messages are summed into dst with no normalisation, a zero-length edge
 *   vector gives Y = (Y00, 0, ..., 0), the radial basis is
 *   sin(n pi r / r_c) / r times the p=6 polynomial envelope, the linear has
 *   no bias, and odd (l1+l2+l3) real coefficients (purely imaginary in this
 *   basis) are represented by their imaginary part.
 */
#include <complex.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_MAX_L 12

/* ------------------------------------------------------------------------ */
/* factorials                                                                */
/* ------------------------------------------------------------------------ */
static double fact(int n) {
  double f = 1.0;
  for (int i = 2; i <= n; ++i) f *= (double)i;
  return f;
}

/* ------------------------------------------------------------------------ */
/* Real spherical harmonics                                                  */
/* ------------------------------------------------------------------------ */

/* Associated Legendre function P_l^m(z), m >= 0, including the
 * Condon-Shortley phase (-1)^m, by the standard three-term recursion in l. */
static double legendre_p(int l, int m, double z) {
  double s = sqrt(fmax(0.0, 1.0 - z * z));
  double pmm = 1.0; /* P_m^m = (-1)^m (2m-1)!! s^m */
  for (int i = 1; i <= m; ++i) pmm *= -(double)(2 * i - 1) * s;
  if (l == m) return pmm;
  double pm1 = z * (double)(2 * m + 1) * pmm; /* P_{m+1}^m */
  if (l == m + 1) return pm1;
  double pl = 0.0;
  for (int ll = m + 2; ll <= l; ++ll) {
    pl = ((double)(2 * ll - 1) * z * pm1 - (double)(ll + m - 1) * pmm) / (double)(ll - m);
    pmm = pm1;
    pm1 = pl;
  }
  return pl;
}

/* Index of a real component inside the (lmax+1)^2 vector, in the page's
 * declaration order: per l, first m=0, then (cos, sin) for m = 1..l. */
static int comp_index(int l, int m, int is_sin) {
  if (m == 0) return l * l;
  return l * l + 2 * m - 1 + is_sin;
}

/* Y[(lmax+1)^2] of direction (x,y,z) (not necessarily unit).  Orthonormal on
 * the sphere; Y_l0 = N P_l(cos t); Y_lm,c/s = sqrt2 N_lm P_l^m(cos t) cos/sin(m phi)
 * with N_lm = sqrt((2l+1)/(4 pi) (l-m)!/(l+m)!). */
static void real_sh(int lmax, double x, double y, double z, double* Y) {
  double r = sqrt(x * x + y * y + z * z);
  int K = (lmax + 1) * (lmax + 1);
  for (int k = 0; k < K; ++k) Y[k] = 0.0;
  Y[0] = sqrt(1.0 / (4.0 * M_PI));
  if (r == 0.0) return; /* zero-length edge: only the l=0 component survives */
  double ct = z / r;
  if (ct > 1.0) ct = 1.0;
  if (ct < -1.0) ct = -1.0;
  double phi = atan2(y, x);
  for (int l = 0; l <= lmax; ++l) {
    for (int m = 0; m <= l; ++m) {
      double n = sqrt((2.0 * l + 1.0) / (4.0 * M_PI) * fact(l - m) / fact(l + m));
      double p = legendre_p(l, m, ct);
      if (m == 0) {
        Y[comp_index(l, 0, 0)] = n * p;
      } else {
        Y[comp_index(l, m, 0)] = sqrt(2.0) * n * p * cos((double)m * phi);
        Y[comp_index(l, m, 1)] = sqrt(2.0) * n * p * sin((double)m * phi);
      }
    }
  }
}

int oracle_sh_f64(int64_t E, const double* vec, int lmax, double* Y) {
  if (lmax < 0 || lmax > OR_MAX_L || E < 0) return 1;
  int K = (lmax + 1) * (lmax + 1);
  for (int64_t e = 0; e < E; ++e) real_sh(lmax, vec[3 * e], vec[3 * e + 1], vec[3 * e + 2], Y + e * K);
  return 0;
}

/* float32 inputs are widened exactly to double first. */
static double* widen(const float* a, int64_t n) {
  double* d = (double*)malloc(sizeof(double) * (n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) d[i] = (double)a[i];
  return d;
}

int oracle_sh(int64_t E, const float* vec, int lmax, double* Y) {
  if (E < 0) return 1;
  double* v = widen(vec, 3 * E);
  int rc = oracle_sh_f64(E, v, lmax, Y);
  free(v);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Clebsch-Gordan coefficients                                               */
/* ------------------------------------------------------------------------ */

/* <l1 m1 l2 m2 | l3 m3> by the Racah formula (integer angular momenta). */
double oracle_cg_complex(int l1, int m1, int l2, int m2, int l3, int m3) {
  if (m3 != m1 + m2) return 0.0;
  if (l3 < abs(l1 - l2) || l3 > l1 + l2) return 0.0;
  if (abs(m1) > l1 || abs(m2) > l2 || abs(m3) > l3) return 0.0;
  double pre = sqrt((2.0 * l3 + 1.0) * fact(l1 + l2 - l3) * fact(l1 - l2 + l3) * fact(-l1 + l2 + l3) /
                    fact(l1 + l2 + l3 + 1));
  pre *= sqrt(fact(l1 + m1) * fact(l1 - m1) * fact(l2 + m2) * fact(l2 - m2) * fact(l3 + m3) * fact(l3 - m3));
  double sum = 0.0;
  for (int k = 0; k <= l1 + l2 + l3; ++k) {
    int a = l1 + l2 - l3 - k, b = l1 - m1 - k, c = l2 + m2 - k;
    int d = l3 - l2 + m1 + k, e = l3 - l1 - m2 + k;
    if (a < 0 || b < 0 || c < 0 || d < 0 || e < 0) continue;
    double den = fact(k) * fact(a) * fact(b) * fact(c) * fact(d) * fact(e);
    sum += ((k & 1) ? -1.0 : 1.0) / den;
  }
  return pre * sum;
}

/* Row mu (page order within l) of the unitary U_l that maps complex SH to
 * real SH: Yreal_mu = sum_m U[mu][m] Y_l^m.  Fills u[2l+1] indexed by m+l. */
static void u_row(int l, int mu, double complex* u) {
  for (int i = 0; i < 2 * l + 1; ++i) u[i] = 0.0;
  if (mu == 0) {
    u[l] = 1.0;
    return;
  }
  int m = (mu + 1) / 2;
  int is_sin = (mu % 2 == 0);
  double sgn = (m & 1) ? -1.0 : 1.0;
  double h = 1.0 / sqrt(2.0);
  if (!is_sin) {
    u[l + m] = h;
    u[l - m] = sgn * h;
  } else {
    u[l + m] = -I * h;
    u[l - m] = I * sgn * h;
  }
}

/* Real-basis coefficients C[mu1][mu2][mu3] for one (l1,l2,l3) triple, with
 * mu in page order.  C = sum U_l3[mu3,m3] <l1m1 l2m2|l3m3> conj(U_l1[mu1,m1])
 * conj(U_l2[mu2,m2]).  For even l1+l2+l3 the result is real; for odd it is
 * purely imaginary and its imaginary part is returned.  Returns -1 if the
 * triple is not allowed, else 0 (real) or 1 (imaginary part taken).  If
 * max_discard is non-NULL it receives the largest magnitude of the discarded
 * (should-be-zero) part. */
int oracle_cg_real(int l1, int l2, int l3, double* out, double* max_discard) {
  if (l1 < 0 || l2 < 0 || l3 < 0 || l1 > OR_MAX_L || l2 > OR_MAX_L || l3 > OR_MAX_L) return -1;
  if (l3 < abs(l1 - l2) || l3 > l1 + l2) return -1;
  int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1, n3 = 2 * l3 + 1;
  int odd = (l1 + l2 + l3) & 1;
  double complex u1[2 * OR_MAX_L + 1], u2[2 * OR_MAX_L + 1], u3[2 * OR_MAX_L + 1];
  double disc = 0.0;
  for (int a = 0; a < n1; ++a) {
    u_row(l1, a, u1);
    for (int b = 0; b < n2; ++b) {
      u_row(l2, b, u2);
      for (int c = 0; c < n3; ++c) {
        u_row(l3, c, u3);
        double complex s = 0.0;
        for (int m1 = -l1; m1 <= l1; ++m1)
          for (int m2 = -l2; m2 <= l2; ++m2) {
            int m3 = m1 + m2;
            if (m3 < -l3 || m3 > l3) continue;
            double cg = oracle_cg_complex(l1, m1, l2, m2, l3, m3);
            s += u3[l3 + m3] * cg * conj(u1[l1 + m1]) * conj(u2[l2 + m2]);
          }
        double keep = odd ? cimag(s) : creal(s);
        double drop = odd ? creal(s) : cimag(s);
        if (fabs(drop) > disc) disc = fabs(drop);
        out[(a * n2 + b) * n3 + c] = keep;
      }
    }
  }
  if (max_discard) *max_discard = disc;
  return odd;
}

/* ------------------------------------------------------------------------ */
/* Path sets                                                                 */
/* ------------------------------------------------------------------------ */

/* Paths (l1 = feature l, l2 = SH l, l3 = output l), all <= lmax, triangle
 * allowed; path_set 0 additionally requires l1+l2+l3 even (parity
 * respecting).  Canonical order: lexicographic in (l1,l2,l3). Returns P. */
int oracle_paths(int lmax, int path_set, int32_t* l1l2l3) {
  if (lmax < 0 || lmax > OR_MAX_L || (path_set != 0 && path_set != 1)) return -1;
  int P = 0;
  for (int l1 = 0; l1 <= lmax; ++l1)
    for (int l2 = 0; l2 <= lmax; ++l2)
      for (int l3 = 0; l3 <= lmax; ++l3) {
        if (l3 < abs(l1 - l2) || l3 > l1 + l2) continue;
        if (path_set == 0 && ((l1 + l2 + l3) & 1)) continue;
        if (l1l2l3) {
          l1l2l3[3 * P] = l1;
          l1l2l3[3 * P + 1] = l2;
          l1l2l3[3 * P + 2] = l3;
        }
        ++P;
      }
  return P;
}

/* ------------------------------------------------------------------------ */
/* Radial weights                                                            */
/* ------------------------------------------------------------------------ */

/* Polynomial envelope with p = 6: u(d) = 1 - 28 d^6 + 48 d^7 - 21 d^8 for
 * d < 1, else 0. */
double oracle_envelope(double d) {
  if (d >= 1.0) return 0.0;
  double d6 = d * d * d * d * d * d;
  return 1.0 - 28.0 * d6 + 48.0 * d6 * d - 21.0 * d6 * d * d;
}

/* Radial basis R_n(r) = sin(n pi r / r_c) / r * u(r / r_c), n = 1..n_basis;
 * at r = 0 the limit n pi / r_c is used. */
void oracle_radial_basis(double r, double r_cut, int n_basis, double* R) {
  double u = oracle_envelope(r / r_cut);
  for (int n = 1; n <= n_basis; ++n) {
    double b = (r == 0.0) ? (double)n * M_PI / r_cut : sin((double)n * M_PI * r / r_cut) / r;
    R[n - 1] = b * u;
  }
}

/* ------------------------------------------------------------------------ */
/* Convolution                                                               */
/* ------------------------------------------------------------------------ */

/* Worker threads of the loops below that run over independent outputs
 * (destination rows, nodes, edges); 0 = the OpenMP default (OMP_NUM_THREADS,
 * else every core of the process).  Splitting the rows over threads changes
 * no sum: each output element still receives its terms in the same order. */
static int g_threads = 0;

void oracle_set_threads(int n) { g_threads = n > 0 ? n : 0; }

int oracle_num_threads(void) {
#ifdef _OPENMP
  return g_threads > 0 ? g_threads : omp_get_max_threads();
#else
  return 1;
#endif
}

/* The coupling blocks of every path, dense, from oracle_cg_real. */
typedef struct {
  int P;
  int32_t* paths; /* [P, 3] (l1, l2, l3) */
  double** cg;    /* cg[p]: [2l1+1][2l2+1][2l3+1] */
} path_blocks;

static int path_blocks_make(int lmax, int path_set, path_blocks* pb) {
  pb->P = oracle_paths(lmax, path_set, NULL);
  if (pb->P <= 0) return 1;
  pb->paths = (int32_t*)malloc(sizeof(int32_t) * 3 * pb->P);
  oracle_paths(lmax, path_set, pb->paths);
  pb->cg = (double**)malloc(sizeof(double*) * pb->P);
  for (int p = 0; p < pb->P; ++p) {
    int l1 = pb->paths[3 * p], l2 = pb->paths[3 * p + 1], l3 = pb->paths[3 * p + 2];
    pb->cg[p] = (double*)malloc(sizeof(double) * (2 * l1 + 1) * (2 * l2 + 1) * (2 * l3 + 1));
    oracle_cg_real(l1, l2, l3, pb->cg[p], NULL);
  }
  return 0;
}

static void path_blocks_free(path_blocks* pb) {
  for (int p = 0; p < pb->P; ++p) free(pb->cg[p]);
  free(pb->cg);
  free(pb->paths);
}

/* Adds edge e's message into the C*K values at o (the destination's block, or
 * the edge's own message block):
 *   o[c, l3 mu3] += sum_p w_e[p,c] sum_{mu1,mu2} C^p[mu1,mu2,mu3] x[src_e, c, l1 mu1] Y_{l2 mu2}(vec_e)
 * in the order: harmonics, per-edge path weights, then paths, mu1, mu2, mu3,
 * channel.  Y [K] and we [P*C] are the caller's work space.  The path
 * weights: weight_mode 0 w[p*C+c]; 1 sum_n R_n(|vec_e|) w[n*P*C + p*C+c];
 * 2 sum_n phi[e*n_basis + n] w[n*P*C + p*C+c] (a given per-edge basis). */
static void edge_message_add(const path_blocks* pb, int lmax, int C, int weight_mode, double r_cut, int n_basis,
                             const double* vec, int64_t e, int64_t s, const double* x, const double* w, double* Y,
                             double* we, double* o, const double* phi) {
  int K = (lmax + 1) * (lmax + 1);
  int P = pb->P;
  double R[64];
  double vx = vec[3 * e], vy = vec[3 * e + 1], vz = vec[3 * e + 2];
  /* 1. spherical harmonics of the edge direction */
  real_sh(lmax, vx, vy, vz, Y);
  /* 2. per-edge path weights */
  if (weight_mode == 0) {
    for (int i = 0; i < P * C; ++i) we[i] = w[i];
  } else if (weight_mode == 2) {
    for (int i = 0; i < P * C; ++i) {
      double acc = 0.0;
      for (int n = 0; n < n_basis; ++n) acc += phi[e * n_basis + n] * w[(int64_t)n * P * C + i];
      we[i] = acc;
    }
  } else {
    double r = sqrt(vx * vx + vy * vy + vz * vz);
    oracle_radial_basis(r, r_cut, n_basis, R);
    for (int i = 0; i < P * C; ++i) {
      double acc = 0.0;
      for (int n = 0; n < n_basis; ++n) acc += R[n] * w[(int64_t)n * P * C + i];
      we[i] = acc;
    }
  }
  /* 3. tensor product with the source features */
  for (int p = 0; p < P; ++p) {
    int l1 = pb->paths[3 * p], l2 = pb->paths[3 * p + 1], l3 = pb->paths[3 * p + 2];
    int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1, n3 = 2 * l3 + 1;
    for (int a = 0; a < n1; ++a)
      for (int b = 0; b < n2; ++b)
        for (int c3 = 0; c3 < n3; ++c3) {
          double coef = pb->cg[p][(a * n2 + b) * n3 + c3];
          if (coef == 0.0) continue;
          double cy = coef * Y[l2 * l2 + b];
          for (int ch = 0; ch < C; ++ch) {
            double xv = x[(s * C + ch) * K + l1 * l1 + a];
            o[ch * K + l3 * l3 + c3] += we[p * C + ch] * cy * xv;
          }
        }
  }
}

/* out[n, c, l3 mu3] = sum_{e: dst_e = n} sum_{p=(l1,l2,l3)} w_e[p,c]
 *                     sum_{mu1,mu2} C^p[mu1,mu2,mu3] x[src_e, c, l1 mu1] Y_{l2 mu2}(vec_e)
 * weight_mode 0: w_e[p,c] = w[p*C + c]   (w is [P, C])
 * weight_mode 1: w_e[p,c] = sum_n R_n(|vec_e|) w[n*P*C + p*C + c]   (w is [n_basis, P*C])
 * x is [N, C, K], out is [N, C, K] float64 and is overwritten.
 * Edges may come in any order; each destination receives its edges' messages
 * in the order given (the edges are grouped by destination, stably, and the
 * destinations are shared out over the threads).  Returns 0 on success,
 * 1 on bad arguments, 2 if an index is out of range (out is then all zero). */
static int conv_core(int64_t N, int64_t E, int lmax, int C, int path_set, int weight_mode, double r_cut,
                     int n_basis, const double* vec, const int32_t* src, const int32_t* dst, const double* x,
                     const double* w, double* out, const double* phi);

int oracle_conv_f64(int64_t N, int64_t E, int lmax, int C, int path_set, int weight_mode, double r_cut,
                    int n_basis, const double* vec, const int32_t* src, const int32_t* dst, const double* x,
                    const double* w, double* out) {
  if (weight_mode != 0 && weight_mode != 1) return 1;
  return conv_core(N, E, lmax, C, path_set, weight_mode, r_cut, n_basis, vec, src, dst, x, w, out, NULL);
}

static int conv_core(int64_t N, int64_t E, int lmax, int C, int path_set, int weight_mode, double r_cut,
                     int n_basis, const double* vec, const int32_t* src, const int32_t* dst, const double* x,
                     const double* w, double* out, const double* phi) {
  if (lmax < 0 || lmax > OR_MAX_L || C <= 0 || N < 0 || E < 0) return 1;
  if (weight_mode == 1 && (n_basis <= 0 || n_basis > 64 || !(r_cut > 0.0))) return 1;
  if (weight_mode == 2 && (n_basis <= 0 || (E > 0 && !phi))) return 1;
  int K = (lmax + 1) * (lmax + 1);
  for (int64_t i = 0; i < N * C * K; ++i) out[i] = 0.0;
  for (int64_t e = 0; e < E; ++e)
    if (src[e] < 0 || src[e] >= N || dst[e] < 0 || dst[e] >= N) return 2;
  path_blocks pb;
  if (path_blocks_make(lmax, path_set, &pb)) return 1;
  int P = pb.P;
  /* edges grouped by destination, in their given order inside each group */
  int64_t* start = (int64_t*)calloc((size_t)N + 1, sizeof(int64_t));
  int64_t* order = (int64_t*)malloc(sizeof(int64_t) * (E > 0 ? E : 1));
  for (int64_t e = 0; e < E; ++e) start[dst[e] + 1]++;
  for (int64_t n = 0; n < N; ++n) start[n + 1] += start[n];
  int64_t* fill = (int64_t*)malloc(sizeof(int64_t) * (N > 0 ? N : 1));
  for (int64_t n = 0; n < N; ++n) fill[n] = start[n];
  for (int64_t e = 0; e < E; ++e) order[fill[dst[e]]++] = e;
  free(fill);
#pragma omp parallel num_threads(oracle_num_threads())
  {
    double* Y = (double*)malloc(sizeof(double) * K);
    double* we = (double*)malloc(sizeof(double) * P * C);
#pragma omp for schedule(dynamic, 16)
    for (int64_t n = 0; n < N; ++n)
      for (int64_t i = start[n]; i < start[n + 1]; ++i) {
        int64_t e = order[i];
        edge_message_add(&pb, lmax, C, weight_mode, r_cut, n_basis, vec, e, src[e], x, w, Y, we,
                         out + n * C * K, phi);
      }
    free(Y);
    free(we);
  }
  free(start);
  free(order);
  path_blocks_free(&pb);
  return 0;
}

/* Per-edge messages (the Batmobile page's fused kernel output, section "3.
 * operator fusion": one [C, K] message per edge, no destination sum):
 *   msg[e, c, l3 m3] = sum_p w_e[p,c] sum_{m1,m2} C^p[m1,m2,m3] x[src_e, c, l1 m1] Y_{l2 m2}(vec_e)
 * with w_e as in oracle_conv_f64.  msg is [E, C, K] float64, overwritten.
 * Returns 2 (msg all zero) if a source index is out of range. */
int oracle_messages_f64(int64_t N, int64_t E, int lmax, int C, int path_set, int weight_mode, double r_cut,
                        int n_basis, const double* vec, const int32_t* src, const double* x, const double* w,
                        double* msg) {
  if (lmax < 0 || lmax > OR_MAX_L || C <= 0 || N < 0 || E < 0) return 1;
  if (weight_mode != 0 && weight_mode != 1) return 1;
  if (weight_mode == 1 && (n_basis <= 0 || n_basis > 64 || !(r_cut > 0.0))) return 1;
  int K = (lmax + 1) * (lmax + 1);
  for (int64_t i = 0; i < E * C * K; ++i) msg[i] = 0.0;
  for (int64_t e = 0; e < E; ++e)
    if (src[e] < 0 || src[e] >= N) return 2;
  path_blocks pb;
  if (path_blocks_make(lmax, path_set, &pb)) return 1;
  int P = pb.P;
#pragma omp parallel num_threads(oracle_num_threads())
  {
    double* Y = (double*)malloc(sizeof(double) * K);
    double* we = (double*)malloc(sizeof(double) * P * C);
#pragma omp for schedule(dynamic, 256)
    for (int64_t e = 0; e < E; ++e)
      edge_message_add(&pb, lmax, C, weight_mode, r_cut, n_basis, vec, e, src[e], x, w, Y, we, msg + e * C * K,
                       NULL);
    free(Y);
    free(we);
  }
  path_blocks_free(&pb);
  return 0;
}

int oracle_messages(int64_t N, int64_t E, int lmax, int C, int path_set, int weight_mode, double r_cut,
                    int n_basis, const float* vec, const int32_t* src, const float* x, const float* w,
                    double* msg) {
  if (lmax < 0 || lmax > OR_MAX_L || C <= 0 || N < 0 || E < 0) return 1;
  int K = (lmax + 1) * (lmax + 1);
  int P = oracle_paths(lmax, path_set, NULL);
  if (P <= 0) return 1;
  if (weight_mode == 1 && (n_basis <= 0 || n_basis > 64)) return 1;
  int64_t nw = (weight_mode == 1) ? (int64_t)n_basis * P * C : (int64_t)P * C;
  double* v = widen(vec, 3 * E);
  double* xx = widen(x, N * C * K);
  double* ww = widen(w, nw);
  int rc = oracle_messages_f64(N, E, lmax, C, path_set, weight_mode, r_cut, n_basis, v, src, xx, ww, msg);
  free(v);
  free(xx);
  free(ww);
  return rc;
}

/* float32 entry point: inputs widened exactly to double, then the f64 core. */
int oracle_conv(int64_t N, int64_t E, int lmax, int C, int path_set, int weight_mode, double r_cut,
                int n_basis, const float* vec, const int32_t* src, const int32_t* dst, const float* x,
                const float* w, double* out) {
  if (lmax < 0 || lmax > OR_MAX_L || C <= 0 || N < 0 || E < 0) return 1;
  int K = (lmax + 1) * (lmax + 1);
  int P = oracle_paths(lmax, path_set, NULL);
  if (P <= 0) return 1;
  int64_t nw = (weight_mode == 1) ? (int64_t)n_basis * P * C : (int64_t)P * C;
  if (weight_mode == 1 && (n_basis <= 0 || n_basis > 64)) return 1;
  double* v = widen(vec, 3 * E);
  double* xx = widen(x, N * C * K);
  double* ww = widen(w, nw);
  int rc = oracle_conv_f64(N, E, lmax, C, path_set, weight_mode, r_cut, n_basis, v, src, dst, xx, ww, out);
  free(v);
  free(xx);
  free(ww);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Gradients of the convolution (fixed weights)                              */
/* ------------------------------------------------------------------------ */

/* Coefficients a[0..l] of the Legendre polynomial P_l(z) = sum_k a_k z^k from
 * the explicit sum P_l(z) = 2^-l sum_j (-1)^j C(l,j) C(2l-2j,l) z^(l-2j). */
static void legendre_coeffs(int l, double* a) {
  for (int k = 0; k <= l; ++k) a[k] = 0.0;
  for (int j = 0; 2 * j <= l; ++j) {
    double c = fact(l) / (fact(j) * fact(l - j)) * fact(2 * l - 2 * j) / (fact(l) * fact(l - 2 * j));
    a[l - 2 * j] += ((j & 1) ? -c : c) / pow(2.0, (double)l);
  }
}

/* m-th derivative of P_l at z (zero for m > l). */
static double legendre_deriv(int l, int m, double z) {
  double a[OR_MAX_L + 2];
  if (m > l) return 0.0;
  legendre_coeffs(l, a);
  double v = 0.0;
  for (int k = l; k >= m; --k) {
    double c = a[k];
    for (int i = 0; i < m; ++i) c *= (double)(k - i); /* d^m/dz^m z^k */
    v = v * z + c;
  }
  /* Horner above ran over k = l..m with powers shifted by m */
  return v;
}

/* Real spherical harmonics and their gradient with respect to the (not
 * normalised) vector v, by a second route independent of real_sh: on the unit
 * sphere u = v/|v| = (x, y, z),
 *   Y_l0     = N_l0 P_l(z),
 *   Y_lm,c/s = sqrt2 N_lm (-1)^m P_l^(m)(z) Re/Im (x + i y)^m,   m = 1..l,
 * (P_l^(m): m-th derivative of the Legendre polynomial; (-1)^m is the
 * Condon-Shortley phase).  These are polynomials in (x, y, z); their gradient
 * g_u is taken componentwise and projected on the sphere's tangent plane:
 * dY/dv = (g_u - u (u . g_u)) / |v|.  G[k*3 + a] = dY_k/dv_a.  A zero vector
 * gives Y = (Y00, 0, ...) and G = 0 (Y is constant there by the reading of
 * the zero-length edge). */
static void real_sh_grad(int lmax, double vx, double vy, double vz, double* Y, double* G) {
  int K = (lmax + 1) * (lmax + 1);
  for (int k = 0; k < K; ++k) {
    Y[k] = 0.0;
    G[3 * k] = G[3 * k + 1] = G[3 * k + 2] = 0.0;
  }
  Y[0] = sqrt(1.0 / (4.0 * M_PI));
  double r = sqrt(vx * vx + vy * vy + vz * vz);
  if (r == 0.0) return;
  double u[3] = {vx / r, vy / r, vz / r};
  double A[OR_MAX_L + 1], B[OR_MAX_L + 1]; /* (x + i y)^m = A_m + i B_m */
  A[0] = 1.0;
  B[0] = 0.0;
  for (int m = 1; m <= lmax; ++m) {
    A[m] = u[0] * A[m - 1] - u[1] * B[m - 1];
    B[m] = u[0] * B[m - 1] + u[1] * A[m - 1];
  }
  for (int l = 0; l <= lmax; ++l) {
    for (int m = 0; m <= l; ++m) {
      double n = sqrt((2.0 * l + 1.0) / (4.0 * M_PI) * fact(l - m) / fact(l + m));
      double D = legendre_deriv(l, m, u[2]), D1 = legendre_deriv(l, m + 1, u[2]);
      double fc, fs, gc[3], gs[3];
      if (m == 0) {
        fc = n * D;
        gc[0] = 0.0;
        gc[1] = 0.0;
        gc[2] = n * D1;
        fs = 0.0;
        gs[0] = gs[1] = gs[2] = 0.0;
      } else {
        double pre = sqrt(2.0) * n * ((m & 1) ? -1.0 : 1.0);
        fc = pre * D * A[m];
        fs = pre * D * B[m];
        /* d/dx (x+iy)^m = m (x+iy)^(m-1), d/dy (x+iy)^m = i m (x+iy)^(m-1) */
        gc[0] = pre * D * m * A[m - 1];
        gc[1] = -pre * D * m * B[m - 1];
        gc[2] = pre * D1 * A[m];
        gs[0] = pre * D * m * B[m - 1];
        gs[1] = pre * D * m * A[m - 1];
        gs[2] = pre * D1 * B[m];
      }
      for (int t = 0; t < 2; ++t) {
        if (m == 0 && t == 1) break;
        int k = comp_index(l, m, t);
        double* g = t ? gs : gc;
        Y[k] = t ? fs : fc;
        double ug = u[0] * g[0] + u[1] * g[1] + u[2] * g[2];
        for (int a = 0; a < 3; ++a) G[3 * k + a] = (g[a] - u[a] * ug) / r;
      }
    }
  }
}

int oracle_sh_grad_f64(int64_t E, const double* vec, int lmax, double* Y, double* G) {
  if (lmax < 0 || lmax > OR_MAX_L || E < 0) return 1;
  int K = (lmax + 1) * (lmax + 1);
  for (int64_t e = 0; e < E; ++e)
    real_sh_grad(lmax, vec[3 * e], vec[3 * e + 1], vec[3 * e + 2], Y + e * K, G + e * K * 3);
  return 0;
}

/* Gradients of L = sum_{n,c,k} gout[n,c,k] out[n,c,k] for the fixed-weight
 * convolution (weight_mode 0) of oracle_conv_f64, written out from its
 * definition term by term:
 *   gx[s,c,l1 m1] = sum_{e: src_e = s} sum_p w[p,c] sum C^p[m1,m2,m3] Y_e[l2 m2] gout[dst_e,c,l3 m3]
 *   gw[p,c]       = sum_e sum C^p[m1,m2,m3] x[src_e,c,l1 m1] Y_e[l2 m2] gout[dst_e,c,l3 m3]
 *   gvec[e]       = sum_k dL/dY_e[k] * dY_k/dvec_e,
 *   dL/dY_e[l2 m2] = sum_c sum_p w[p,c] sum C^p[m1,m2,m3] x[src_e,c,l1 m1] gout[dst_e,c,l3 m3].
 * Y comes from real_sh (as in the forward), dY/dvec from real_sh_grad.
 * Any of gx [N,C,K], gw [P,C], gvec [E,3] may be NULL; the others are
 * overwritten.  Returns 0 on success. */
int oracle_conv_backward_f64(int64_t N, int64_t E, int lmax, int C, int path_set, const double* vec,
                             const int32_t* src, const int32_t* dst, const double* x, const double* w,
                             const double* gout, double* gx, double* gw, double* gvec) {
  if (lmax < 0 || lmax > OR_MAX_L || C <= 0 || N < 0 || E < 0) return 1;
  int K = (lmax + 1) * (lmax + 1);
  int P = oracle_paths(lmax, path_set, NULL);
  if (P <= 0) return 1;
  int32_t* paths = (int32_t*)malloc(sizeof(int32_t) * 3 * P);
  oracle_paths(lmax, path_set, paths);
  double** cg = (double**)malloc(sizeof(double*) * P);
  for (int p = 0; p < P; ++p) {
    int l1 = paths[3 * p], l2 = paths[3 * p + 1], l3 = paths[3 * p + 2];
    cg[p] = (double*)malloc(sizeof(double) * (2 * l1 + 1) * (2 * l2 + 1) * (2 * l3 + 1));
    oracle_cg_real(l1, l2, l3, cg[p], NULL);
  }
  if (gx)
    for (int64_t i = 0; i < N * C * K; ++i) gx[i] = 0.0;
  if (gw)
    for (int64_t i = 0; i < (int64_t)P * C; ++i) gw[i] = 0.0;
  double* Y = (double*)malloc(sizeof(double) * K);
  double* Y2 = (double*)malloc(sizeof(double) * K);
  double* G = (double*)malloc(sizeof(double) * K * 3);
  double* dY = (double*)malloc(sizeof(double) * K);
  int rc = 0;
  for (int64_t e = 0; e < E; ++e) {
    int64_t s = src[e], d = dst[e];
    if (s < 0 || s >= N || d < 0 || d >= N) {
      rc = 2;
      break;
    }
    double vx = vec[3 * e], vy = vec[3 * e + 1], vz = vec[3 * e + 2];
    real_sh(lmax, vx, vy, vz, Y);
    real_sh_grad(lmax, vx, vy, vz, Y2, G);
    for (int k = 0; k < K; ++k) dY[k] = 0.0;
    for (int p = 0; p < P; ++p) {
      int l1 = paths[3 * p], l2 = paths[3 * p + 1], l3 = paths[3 * p + 2];
      int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1, n3 = 2 * l3 + 1;
      for (int a = 0; a < n1; ++a)
        for (int b = 0; b < n2; ++b)
          for (int c3 = 0; c3 < n3; ++c3) {
            double coef = cg[p][(a * n2 + b) * n3 + c3];
            if (coef == 0.0) continue;
            for (int ch = 0; ch < C; ++ch) {
              double xv = x[(s * C + ch) * K + l1 * l1 + a];
              double gv = gout[(d * C + ch) * K + l3 * l3 + c3];
              double wv = w[p * C + ch];
              double yv = Y[l2 * l2 + b];
              if (gx) gx[(s * C + ch) * K + l1 * l1 + a] += wv * coef * yv * gv;
              if (gw) gw[p * C + ch] += coef * xv * yv * gv;
              dY[l2 * l2 + b] += wv * coef * xv * gv;
            }
          }
    }
    if (gvec)
      for (int a = 0; a < 3; ++a) {
        double acc = 0.0;
        for (int k = 0; k < K; ++k) acc += dY[k] * G[3 * k + a];
        gvec[3 * e + a] = acc;
      }
  }
  free(Y);
  free(Y2);
  free(G);
  free(dY);
  for (int p = 0; p < P; ++p) free(cg[p]);
  free(cg);
  free(paths);
  return rc;
}

/* float32 entry point: inputs widened exactly to double. */
int oracle_conv_backward(int64_t N, int64_t E, int lmax, int C, int path_set, const float* vec,
                         const int32_t* src, const int32_t* dst, const float* x, const float* w,
                         const float* gout, double* gx, double* gw, double* gvec) {
  if (lmax < 0 || lmax > OR_MAX_L || C <= 0 || N < 0 || E < 0) return 1;
  int K = (lmax + 1) * (lmax + 1);
  int P = oracle_paths(lmax, path_set, NULL);
  if (P <= 0) return 1;
  double* v = widen(vec, 3 * E);
  double* xx = widen(x, N * C * K);
  double* ww = widen(w, (int64_t)P * C);
  double* gg = widen(gout, N * C * K);
  int rc = oracle_conv_backward_f64(N, E, lmax, C, path_set, v, src, dst, xx, ww, gg, gx, gw, gvec);
  free(v);
  free(xx);
  free(ww);
  free(gg);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Gradients of the convolution with radial weights                          */
/* ------------------------------------------------------------------------ */

/* Derivative of the p = 6 envelope: u'(d) = -168 d^5 + 336 d^6 - 168 d^7 for
 * d < 1, else 0 (u, u' and u'' all vanish at d = 1). */
double oracle_envelope_deriv(double d) {
  if (d >= 1.0) return 0.0;
  double d5 = d * d * d * d * d;
  return -168.0 * d5 + 336.0 * d5 * d - 168.0 * d5 * d * d;
}

/* dR_n/dr of oracle_radial_basis, n = 1..n_basis: with a = n pi / r_c,
 *   d/dr [sin(a r)/r u(r/r_c)] = (a r cos(a r) - sin(a r)) / r^2 u(r/r_c) + sin(a r)/r u'(r/r_c) / r_c.
 * For a r < 1e-2 the first quotient (a difference of nearly equal terms over
 * a vanishing r^2) is taken from its Taylor series
 * -a^3 r / 3 + a^5 r^3 / 30 - a^7 r^5 / 840 (next term a^9 r^7 / 45360, below
 * 1e-16 relative there); at r = 0 it is 0, and so is u'(0), so dR = 0.
 * Likewise sin(a r)/r is taken as a for r = 0. */
void oracle_radial_basis_deriv(double r, double r_cut, int n_basis, double* dR) {
  double d = r / r_cut;
  double u = oracle_envelope(d), du = oracle_envelope_deriv(d) / r_cut;
  for (int n = 1; n <= n_basis; ++n) {
    double a = (double)n * M_PI / r_cut;
    double ar = a * r;
    double ds, s;
    if (ar < 1e-2) {
      double a3r = a * a * a * r, ar2 = ar * ar;
      ds = -a3r / 3.0 + a3r * ar2 / 30.0 - a3r * ar2 * ar2 / 840.0;
      s = r == 0.0 ? a : sin(ar) / r;
    } else {
      ds = (ar * cos(ar) - sin(ar)) / (r * r);
      s = sin(ar) / r;
    }
    dR[n - 1] = ds * u + s * du;
  }
}

#define OR_BWD_BLOCK 1024 /* source nodes per partial sum of grad_W */

/* Gradients of L = sum_{n,c,k} gout[n,c,k] out[n,c,k] for the radial-weight
 * convolution (weight_mode 1 of oracle_conv_f64), where edge e = (s -> d) has
 * the path weights w_e[p,c] = sum_b R_b(r_e) W[b, p*C + c], r_e = |vec_e|:
 *   gx[s,c,l1 m1]  = sum_{e: src_e = s} sum_p w_e[p,c] sum_{m2,m3} C^p Y_e[l2 m2] gout[d,c,l3 m3]
 *   T_e[p,c]       = sum_{m1,m2,m3} C^p x[s,c,l1 m1] Y_e[l2 m2] gout[d,c,l3 m3]   (dL/dw_e[p,c])
 *   gW[b, p*C + c] = sum_e R_b(r_e) T_e[p,c]
 *   dL/dY_e[l2 m2] = sum_c sum_p w_e[p,c] sum_{m1,m3} C^p x[s,c,l1 m1] gout[d,c,l3 m3]
 *   dL/dR_b(e)     = sum_{p,c} W[b, p*C + c] T_e[p,c]
 *   gvec[e]        = sum_k dL/dY_e[k] dY_k/dvec_e + (sum_b dL/dR_b(e) R_b'(r_e)) vec_e / r_e
 * (the last term is 0 for a zero-length edge).  gW is [n_basis, P*C].  The
 * edges are grouped by source, stably; blocks of OR_BWD_BLOCK source nodes are
 * shared out over the threads, each block sums its edges' gW terms in order
 * into a partial of its own, and the partials are added in block order, so
 * the result does not depend on the thread count.  Any of gx, gW, gvec may
 * be NULL.  Returns 0, 1 on bad arguments, 2 if an index is out of range
 * (the requested outputs are then zero). */
int oracle_conv_backward_radial_f64(int64_t N, int64_t E, int lmax, int C, int path_set, double r_cut,
                                    int n_basis, const double* vec, const int32_t* src, const int32_t* dst,
                                    const double* x, const double* W, const double* gout, double* gx, double* gW,
                                    double* gvec) {
  if (lmax < 0 || lmax > OR_MAX_L || C <= 0 || N < 0 || E < 0) return 1;
  if (n_basis <= 0 || n_basis > 64 || !(r_cut > 0.0)) return 1;
  int K = (lmax + 1) * (lmax + 1);
  path_blocks pb;
  if (path_blocks_make(lmax, path_set, &pb)) return 1;
  int P = pb.P;
  int64_t PC = (int64_t)P * C;
  if (gx)
    for (int64_t i = 0; i < N * C * K; ++i) gx[i] = 0.0;
  if (gW)
    for (int64_t i = 0; i < n_basis * PC; ++i) gW[i] = 0.0;
  if (gvec)
    for (int64_t i = 0; i < 3 * E; ++i) gvec[i] = 0.0;
  for (int64_t e = 0; e < E; ++e)
    if (src[e] < 0 || src[e] >= N || dst[e] < 0 || dst[e] >= N) {
      path_blocks_free(&pb);
      return 2;
    }
  /* edges grouped by source, in their given order inside each group */
  int64_t* start = (int64_t*)calloc((size_t)N + 1, sizeof(int64_t));
  int64_t* order = (int64_t*)malloc(sizeof(int64_t) * (E > 0 ? E : 1));
  int64_t* fill = (int64_t*)malloc(sizeof(int64_t) * (N > 0 ? N : 1));
  for (int64_t e = 0; e < E; ++e) start[src[e] + 1]++;
  for (int64_t n = 0; n < N; ++n) start[n + 1] += start[n];
  for (int64_t n = 0; n < N; ++n) fill[n] = start[n];
  for (int64_t e = 0; e < E; ++e) order[fill[src[e]]++] = e;
  free(fill);
  int64_t nblk = (N + OR_BWD_BLOCK - 1) / OR_BWD_BLOCK;
  double* part = gW ? (double*)calloc((size_t)(nblk > 0 ? nblk : 1) * n_basis * PC, sizeof(double)) : NULL;
#pragma omp parallel num_threads(oracle_num_threads())
  {
    double* Y = (double*)malloc(sizeof(double) * K);
    double* Y2 = (double*)malloc(sizeof(double) * K);
    double* G = (double*)malloc(sizeof(double) * K * 3);
    double* dY = (double*)malloc(sizeof(double) * K);
    double* we = (double*)malloc(sizeof(double) * PC);
    double* T = (double*)malloc(sizeof(double) * PC);
    double R[64], dR[64];
#pragma omp for schedule(dynamic, 1)
    for (int64_t blk = 0; blk < nblk; ++blk) {
      int64_t n_end = (blk + 1) * OR_BWD_BLOCK < N ? (blk + 1) * OR_BWD_BLOCK : N;
      for (int64_t i = start[blk * OR_BWD_BLOCK]; i < start[n_end]; ++i) {
        int64_t e = order[i];
        int64_t s = src[e], d = dst[e];
        double vx = vec[3 * e], vy = vec[3 * e + 1], vz = vec[3 * e + 2];
        double r = sqrt(vx * vx + vy * vy + vz * vz);
        /* radial functions, path weights and harmonics of the edge */
        oracle_radial_basis(r, r_cut, n_basis, R);
        oracle_radial_basis_deriv(r, r_cut, n_basis, dR);
        for (int64_t q = 0; q < PC; ++q) {
          double acc = 0.0;
          for (int b = 0; b < n_basis; ++b) acc += R[b] * W[b * PC + q];
          we[q] = acc;
          T[q] = 0.0;
        }
        real_sh(lmax, vx, vy, vz, Y);
        real_sh_grad(lmax, vx, vy, vz, Y2, G);
        for (int k = 0; k < K; ++k) dY[k] = 0.0;
        /* the coupling, term by term */
        for (int p = 0; p < P; ++p) {
          int l1 = pb.paths[3 * p], l2 = pb.paths[3 * p + 1], l3 = pb.paths[3 * p + 2];
          int n1 = 2 * l1 + 1, n2 = 2 * l2 + 1, n3 = 2 * l3 + 1;
          for (int a = 0; a < n1; ++a)
            for (int b2 = 0; b2 < n2; ++b2)
              for (int c3 = 0; c3 < n3; ++c3) {
                double coef = pb.cg[p][(a * n2 + b2) * n3 + c3];
                if (coef == 0.0) continue;
                for (int ch = 0; ch < C; ++ch) {
                  double xv = x[(s * C + ch) * K + l1 * l1 + a];
                  double gv = gout[(d * C + ch) * K + l3 * l3 + c3];
                  double yv = Y[l2 * l2 + b2];
                  double wv = we[p * C + ch];
                  if (gx) gx[(s * C + ch) * K + l1 * l1 + a] += wv * coef * yv * gv;
                  T[p * C + ch] += coef * xv * yv * gv;
                  dY[l2 * l2 + b2] += wv * coef * xv * gv;
                }
              }
        }
        /* grad_W: this block's partial */
        if (part)
          for (int b = 0; b < n_basis; ++b)
            for (int64_t q = 0; q < PC; ++q) part[(blk * n_basis + b) * PC + q] += R[b] * T[q];
        if (gvec) {
          double dr = 0.0; /* dL/dr_e */
          for (int b = 0; b < n_basis; ++b) {
            double dLdR = 0.0;
            for (int64_t q = 0; q < PC; ++q) dLdR += W[b * PC + q] * T[q];
            dr += dLdR * dR[b];
          }
          for (int ax = 0; ax < 3; ++ax) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k) acc += dY[k] * G[3 * k + ax];
            if (r > 0.0) acc += dr * vec[3 * e + ax] / r;
            gvec[3 * e + ax] = acc;
          }
        }
      }
    }
    free(Y);
    free(Y2);
    free(G);
    free(dY);
    free(we);
    free(T);
  }
  if (gW)
    for (int64_t blk = 0; blk < nblk; ++blk)
      for (int64_t q = 0; q < n_basis * PC; ++q) gW[q] += part[blk * n_basis * PC + q];
  free(part);
  free(start);
  free(order);
  path_blocks_free(&pb);
  return 0;
}

/* float32 entry point: inputs widened exactly to double. */
int oracle_conv_backward_radial(int64_t N, int64_t E, int lmax, int C, int path_set, double r_cut, int n_basis,
                                const float* vec, const int32_t* src, const int32_t* dst, const float* x,
                                const float* W, const float* gout, double* gx, double* gW, double* gvec) {
  if (lmax < 0 || lmax > OR_MAX_L || C <= 0 || N < 0 || E < 0) return 1;
  if (n_basis <= 0 || n_basis > 64) return 1;
  int K = (lmax + 1) * (lmax + 1);
  int P = oracle_paths(lmax, path_set, NULL);
  if (P <= 0) return 1;
  double* v = widen(vec, 3 * E);
  double* xx = widen(x, N * C * K);
  double* ww = widen(W, (int64_t)n_basis * P * C);
  double* gg = widen(gout, N * C * K);
  int rc = oracle_conv_backward_radial_f64(N, E, lmax, C, path_set, r_cut, n_basis, v, src, dst, xx, ww, gg, gx,
                                           gW, gvec);
  free(v);
  free(xx);
  free(ww);
  free(gg);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Per-l channel linear                                                      */
/* ------------------------------------------------------------------------ */

/* Round a float32 to the nearest bfloat16 (ties to even) and return it as a
 * float32 value.  NaN is kept as a quiet NaN. */
static float round_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) {
    u |= 0x00400000u;
    u &= 0xffff0000u;
  } else {
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    u &= 0xffff0000u;
  }
  float r;
  memcpy(&r, &u, 4);
  return r;
}

float oracle_round_bf16(float f) { return round_bf16(f); }

/* out[n, c', l mu] = sum_c W[l, c', c] h[n, c, l mu] in double precision. */
int oracle_linear_f64(int64_t N, int C, int lmax, const double* h, const double* W, double* out) {
  if (lmax < 0 || lmax > OR_MAX_L || C <= 0 || N < 0) return 1;
  int K = (lmax + 1) * (lmax + 1);
#pragma omp parallel for schedule(static) num_threads(oracle_num_threads())
  for (int64_t n = 0; n < N; ++n)
    for (int l = 0; l <= lmax; ++l)
      for (int mu = l * l; mu < (l + 1) * (l + 1); ++mu)
        for (int co = 0; co < C; ++co) {
          double acc = 0.0;
          for (int ci = 0; ci < C; ++ci) acc += W[((int64_t)l * C + co) * C + ci] * h[(n * C + ci) * K + mu];
          out[(n * C + co) * K + mu] = acc;
        }
  return 0;
}

/* out[n, c', l mu] = sum_c W[l, c', c] h[n, c, l mu], W is [lmax+1, C, C]
 * (output channel major).  If bf16 != 0 both h and W are first rounded to
 * bfloat16 (round to nearest even), as the bf16 matrix-core mode consumes
 * them; products and sums are then exact/fp64 here. */
int oracle_linear(int64_t N, int C, int lmax, int bf16, const float* h, const float* W, double* out) {
  if (lmax < 0 || lmax > OR_MAX_L || C <= 0 || N < 0) return 1;
  int K = (lmax + 1) * (lmax + 1);
#pragma omp parallel for schedule(static) num_threads(oracle_num_threads())
  for (int64_t n = 0; n < N; ++n)
    for (int l = 0; l <= lmax; ++l)
      for (int mu = l * l; mu < (l + 1) * (l + 1); ++mu)
        for (int co = 0; co < C; ++co) {
          double acc = 0.0;
          for (int ci = 0; ci < C; ++ci) {
            float wv = W[((int64_t)l * C + co) * C + ci];
            float hv = h[(n * C + ci) * K + mu];
            if (bf16) {
              wv = round_bf16(wv);
              hv = round_bf16(hv);
            }
            acc += (double)wv * (double)hv;
          }
          out[(n * C + co) * K + mu] = acc;
        }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Interaction layer: channel linear, radial MLP, convolution, channel linear */
/* ------------------------------------------------------------------------ */

/* SiLU(t) = t / (1 + exp(-t)). */
double oracle_silu(double t) { return t / (1.0 + exp(-t)); }

/* The radial network of an edge: R = radial basis of |vec_e| (n_basis
 * functions, as in the radial weights), then two hidden layers of width H
 * with SiLU and no bias:
 *   a[k]      = SiLU(sum_b R_b W1[b*H + k]),
 *   phi[e, k] = SiLU(sum_j a[j] W2[j*H + k]).
 * phi is [E, H]. */
int oracle_radial_mlp_f64(int64_t E, const double* vec, double r_cut, int n_basis, int H, const double* W1,
                          const double* W2, double* phi) {
  if (E < 0 || n_basis <= 0 || n_basis > 64 || H <= 0 || !(r_cut > 0.0)) return 1;
#pragma omp parallel num_threads(oracle_num_threads())
  {
    double R[64];
    double* a = (double*)malloc(sizeof(double) * H);
#pragma omp for schedule(static)
    for (int64_t e = 0; e < E; ++e) {
      double vx = vec[3 * e], vy = vec[3 * e + 1], vz = vec[3 * e + 2];
      oracle_radial_basis(sqrt(vx * vx + vy * vy + vz * vz), r_cut, n_basis, R);
      for (int k = 0; k < H; ++k) {
        double acc = 0.0;
        for (int b = 0; b < n_basis; ++b) acc += R[b] * W1[(int64_t)b * H + k];
        a[k] = oracle_silu(acc);
      }
      for (int k = 0; k < H; ++k) {
        double acc = 0.0;
        for (int j = 0; j < H; ++j) acc += a[j] * W2[(int64_t)j * H + k];
        phi[e * H + k] = oracle_silu(acc);
      }
    }
    free(a);
  }
  return 0;
}

/* The convolution of oracle_conv_f64 with per-edge path weights from a given
 * per-edge basis phi [E, H]: w_e[p,c] = sum_k phi[e,k] W3[k, p*C + c]. */
int oracle_conv_basis_f64(int64_t N, int64_t E, int lmax, int C, int path_set, int H, const double* vec,
                          const int32_t* src, const int32_t* dst, const double* x, const double* phi,
                          const double* W3, double* out) {
  return conv_core(N, E, lmax, C, path_set, 2, 0.0, H, vec, src, dst, x, W3, out, phi);
}

/* One interaction layer on node features h [N, C, K]:
 *   h1  = linear(h, W_up)                       (per-l channel linear, W_up [lmax+1, C, C])
 *   phi = radial MLP of the edge lengths        (oracle_radial_mlp_f64: W1 [n_basis, H], W2 [H, H])
 *   m   = conv of h1 with w_e = phi_e W3        (oracle_conv_basis_f64: W3 [H, P*C])
 *   out = linear(m, W_out) / norm               (W_out [lmax+1, C, C]; norm > 0, e.g. the mean degree)
 * out is [N, C, K]. */
int oracle_interaction_f64(int64_t N, int64_t E, int lmax, int C, int path_set, double r_cut, int n_basis, int H,
                           const double* vec, const int32_t* src, const int32_t* dst, const double* h,
                           const double* W_up, const double* W1, const double* W2, const double* W3,
                           const double* W_out, double norm, double* out) {
  if (lmax < 0 || lmax > OR_MAX_L || C <= 0 || N < 0 || E < 0 || !(norm > 0.0)) return 1;
  int K = (lmax + 1) * (lmax + 1);
  double* h1 = (double*)malloc(sizeof(double) * (N * C * K > 0 ? N * C * K : 1));
  double* m = (double*)malloc(sizeof(double) * (N * C * K > 0 ? N * C * K : 1));
  double* phi = (double*)malloc(sizeof(double) * (E * H > 0 ? E * H : 1));
  int rc = oracle_linear_f64(N, C, lmax, h, W_up, h1);
  if (!rc) rc = oracle_radial_mlp_f64(E, vec, r_cut, n_basis, H, W1, W2, phi);
  if (!rc) rc = oracle_conv_basis_f64(N, E, lmax, C, path_set, H, vec, src, dst, h1, phi, W3, m);
  if (!rc) rc = oracle_linear_f64(N, C, lmax, m, W_out, out);
  if (!rc)
    for (int64_t i = 0; i < N * C * K; ++i) out[i] /= norm;
  free(h1);
  free(m);
  free(phi);
  return rc;
}

/* float32 entry point: inputs widened exactly to double. */
int oracle_interaction(int64_t N, int64_t E, int lmax, int C, int path_set, double r_cut, int n_basis, int H,
                       const float* vec, const int32_t* src, const int32_t* dst, const float* h, const float* W_up,
                       const float* W1, const float* W2, const float* W3, const float* W_out, double norm,
                       double* out) {
  if (lmax < 0 || lmax > OR_MAX_L || C <= 0 || N < 0 || E < 0 || H <= 0 || n_basis <= 0) return 1;
  int K = (lmax + 1) * (lmax + 1);
  int P = oracle_paths(lmax, path_set, NULL);
  if (P <= 0) return 1;
  double* v = widen(vec, 3 * E);
  double* hh = widen(h, N * C * K);
  double* wu = widen(W_up, (int64_t)(lmax + 1) * C * C);
  double* w1 = widen(W1, (int64_t)n_basis * H);
  double* w2 = widen(W2, (int64_t)H * H);
  double* w3 = widen(W3, (int64_t)H * P * C);
  double* wo = widen(W_out, (int64_t)(lmax + 1) * C * C);
  int rc = oracle_interaction_f64(N, E, lmax, C, path_set, r_cut, n_basis, H, v, src, dst, hh, wu, w1, w2, w3, wo,
                                  norm, out);
  free(v);
  free(hh);
  free(wu);
  free(w1);
  free(w2);
  free(w3);
  free(wo);
  return rc;
}
