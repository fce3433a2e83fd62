/*
 * oracle_sanitize_main.c -- test driver that runs every entry point of the
 * CPU oracle (oracle/eqtp_oracle.c) on small seeded inputs, including the
 * degenerate ones (no nodes, no edges, zero-length and polar edge vectors,
 * out-of-range indices, invalid arguments, NaN/inf for the bf16 rounding).
 * It is compiled together with the oracle under AddressSanitizer and
 * UndefinedBehaviorSanitizer by tests/test_oracle_sanitize.py; any invalid
 * access or undefined operation aborts it.  Every buffer is allocated at its
 * exact size so that a read or write past its end is caught.  The checks here
 * are on return codes only; the values are pinned by the other oracle tests.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_sh_f64(int64_t E, const double* vec, int lmax, double* Y);
int oracle_sh(int64_t E, const float* vec, int lmax, double* Y);
double oracle_cg_complex(int l1, int m1, int l2, int m2, int l3, int m3);
int oracle_cg_real(int l1, int l2, int l3, double* out, double* max_discard);
int oracle_paths(int lmax, int path_set, int32_t* l1l2l3);
double oracle_envelope(double d);
void oracle_radial_basis(double r, double r_cut, int n_basis, double* R);
void oracle_set_threads(int n);
int oracle_num_threads(void);
int oracle_conv_f64(int64_t N, int64_t E, int lmax, int C, int path_set, int weight_mode, double r_cut, int n_basis,
                    const double* vec, const int32_t* src, const int32_t* dst, const double* x, const double* w,
                    double* out);
int oracle_messages_f64(int64_t N, int64_t E, int lmax, int C, int path_set, int weight_mode, double r_cut,
                        int n_basis, const double* vec, const int32_t* src, const double* x, const double* w,
                        double* msg);
int oracle_messages(int64_t N, int64_t E, int lmax, int C, int path_set, int weight_mode, double r_cut, int n_basis,
                    const float* vec, const int32_t* src, const float* x, const float* w, double* msg);
int oracle_conv(int64_t N, int64_t E, int lmax, int C, int path_set, int weight_mode, double r_cut, int n_basis,
                const float* vec, const int32_t* src, const int32_t* dst, const float* x, const float* w,
                double* out);
int oracle_sh_grad_f64(int64_t E, const double* vec, int lmax, double* Y, double* G);
int oracle_conv_backward_f64(int64_t N, int64_t E, int lmax, int C, int path_set, const double* vec,
                             const int32_t* src, const int32_t* dst, const double* x, const double* w,
                             const double* gout, double* gx, double* gw, double* gvec);
int oracle_conv_backward(int64_t N, int64_t E, int lmax, int C, int path_set, const float* vec, const int32_t* src,
                         const int32_t* dst, const float* x, const float* w, const float* gout, double* gx,
                         double* gw, double* gvec);
double oracle_envelope_deriv(double d);
void oracle_radial_basis_deriv(double r, double r_cut, int n_basis, double* dR);
int oracle_conv_backward_radial_f64(int64_t N, int64_t E, int lmax, int C, int path_set, double r_cut,
                                    int n_basis, const double* vec, const int32_t* src, const int32_t* dst,
                                    const double* x, const double* W, const double* gout, double* gx, double* gW,
                                    double* gvec);
int oracle_conv_backward_radial(int64_t N, int64_t E, int lmax, int C, int path_set, double r_cut, int n_basis,
                                const float* vec, const int32_t* src, const int32_t* dst, const float* x,
                                const float* W, const float* gout, double* gx, double* gW, double* gvec);
float oracle_round_bf16(float f);
double oracle_silu(double t);
int oracle_radial_mlp_f64(int64_t E, const double* vec, double r_cut, int n_basis, int H, const double* W1,
                          const double* W2, double* phi);
int oracle_conv_basis_f64(int64_t N, int64_t E, int lmax, int C, int path_set, int H, const double* vec,
                          const int32_t* src, const int32_t* dst, const double* x, const double* phi,
                          const double* W3, double* out);
int oracle_interaction(int64_t N, int64_t E, int lmax, int C, int path_set, double r_cut, int n_basis, int H,
                       const float* vec, const int32_t* src, const int32_t* dst, const float* h, const float* W_up,
                       const float* W1, const float* W2, const float* W3, const float* W_out, double norm,
                       double* out);
int oracle_linear_f64(int64_t N, int C, int lmax, const double* h, const double* W, double* out);
int oracle_linear(int64_t N, int C, int lmax, int bf16, const float* h, const float* W, double* out);

static int failures = 0;
#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

/* splitmix64: a seeded stream of uniform numbers, nothing of the method */
static uint64_t rng_state = 0x1234567ull;
static uint64_t next_u64(void) {
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static double uniform(double lo, double hi) { return lo + (hi - lo) * (double)(next_u64() >> 11) * 0x1.0p-53; }
static int32_t index_below(int64_t n) { return (int32_t)(next_u64() % (uint64_t)n); }

static void* xmalloc(size_t bytes) {
  void* p = malloc(bytes > 0 ? bytes : 1);
  if (!p) {
    fprintf(stderr, "out of memory\n");
    exit(3);
  }
  return p;
}

/* edge vectors with the special directions first: zero, +z, -z, +x, -y, tiny */
static void fill_vectors(int64_t E, double* v) {
  static const double special[6][3] = {{0, 0, 0}, {0, 0, 1.5}, {0, 0, -2}, {0.7, 0, 0}, {0, -1, 0}, {1e-30, 0, 1e-30}};
  for (int64_t e = 0; e < E; ++e)
    for (int a = 0; a < 3; ++a) v[3 * e + a] = e < 6 ? special[e][a] : uniform(-3.0, 3.0);
}

static void test_sh(void) {
  for (int lmax = 0; lmax <= 12; ++lmax) {
    const int64_t E = 11;
    const int K = (lmax + 1) * (lmax + 1);
    double* v = (double*)xmalloc(sizeof(double) * 3 * E);
    float* vf = (float*)xmalloc(sizeof(float) * 3 * E);
    double* Y = (double*)xmalloc(sizeof(double) * E * K);
    double* G = (double*)xmalloc(sizeof(double) * E * K * 3);
    fill_vectors(E, v);
    for (int64_t i = 0; i < 3 * E; ++i) vf[i] = (float)v[i];
    EXPECT(oracle_sh_f64(E, v, lmax, Y) == 0);
    EXPECT(oracle_sh(E, vf, lmax, Y) == 0);
    EXPECT(oracle_sh_grad_f64(E, v, lmax, Y, G) == 0);
    EXPECT(oracle_sh_f64(0, v, lmax, Y) == 0);
    for (int64_t i = 0; i < E * K; ++i) EXPECT(isfinite(Y[i]));
    free(v);
    free(vf);
    free(Y);
    free(G);
  }
  EXPECT(oracle_sh_f64(1, NULL, 13, NULL) == 1);
  EXPECT(oracle_sh_f64(-1, NULL, 2, NULL) == 1);
  EXPECT(oracle_sh_grad_f64(1, NULL, -1, NULL, NULL) == 1);
}

static void test_cg_and_paths(void) {
  for (int l1 = 0; l1 <= 4; ++l1)
    for (int l2 = 0; l2 <= 4; ++l2)
      for (int l3 = 0; l3 <= 4; ++l3) {
        const int n = (2 * l1 + 1) * (2 * l2 + 1) * (2 * l3 + 1);
        double* c = (double*)xmalloc(sizeof(double) * n);
        double disc = -1.0;
        const int rc = oracle_cg_real(l1, l2, l3, c, &disc);
        const int allowed = l3 >= abs(l1 - l2) && l3 <= l1 + l2;
        EXPECT(allowed ? (rc == ((l1 + l2 + l3) & 1)) : rc == -1);
        if (allowed) EXPECT(disc >= 0.0 && disc < 1e-12);
        if (allowed) EXPECT(oracle_cg_real(l1, l2, l3, c, NULL) == rc);
        free(c);
        for (int m1 = -l1 - 1; m1 <= l1 + 1; ++m1)
          for (int m2 = -l2 - 1; m2 <= l2 + 1; ++m2) EXPECT(isfinite(oracle_cg_complex(l1, m1, l2, m2, l3, m1 + m2)));
      }
  /* the largest l the oracle accepts, on a small triple and a full one */
  {
    double* c = (double*)xmalloc(sizeof(double) * 25 * 25 * 25);
    EXPECT(oracle_cg_real(12, 12, 0, c, NULL) == 0);
    EXPECT(oracle_cg_real(0, 12, 12, c, NULL) == 0);
    EXPECT(oracle_cg_real(12, 1, 12, c, NULL) == 1);
    free(c);
  }
  EXPECT(oracle_cg_real(13, 0, 13, NULL, NULL) == -1);
  EXPECT(oracle_cg_real(-1, 0, 1, NULL, NULL) == -1);
  for (int lmax = 0; lmax <= 12; ++lmax)
    for (int ps = 0; ps <= 1; ++ps) {
      const int P = oracle_paths(lmax, ps, NULL);
      EXPECT(P > 0);
      int32_t* t = (int32_t*)xmalloc(sizeof(int32_t) * 3 * P);
      EXPECT(oracle_paths(lmax, ps, t) == P);
      free(t);
    }
  EXPECT(oracle_paths(13, 0, NULL) == -1);
  EXPECT(oracle_paths(2, 2, NULL) == -1);
}

static void test_radial(void) {
  double R[64];
  const double rs[] = {0.0, 1e-300, 0.3, 4.999999, 5.0, 7.0};
  for (int i = 0; i < 6; ++i)
    for (int nb = 1; nb <= 64; nb *= 2) {
      oracle_radial_basis(rs[i], 5.0, nb, R);
      for (int b = 0; b < nb; ++b) EXPECT(isfinite(R[b]));
      oracle_radial_basis_deriv(rs[i], 5.0, nb, R);
      for (int b = 0; b < nb; ++b) EXPECT(isfinite(R[b]));
    }
  EXPECT(oracle_envelope(1.0) == 0.0);
  EXPECT(oracle_envelope(0.0) == 1.0);
  EXPECT(oracle_envelope(2.0) == 0.0);
  EXPECT(oracle_envelope_deriv(0.0) == 0.0);
  EXPECT(oracle_envelope_deriv(1.5) == 0.0);
}

/* one convolution case: forward (fp64 and fp32 entry points), messages and,
 * for fixed weights, the backward with every subset of outputs */
static void conv_case(int64_t N, int64_t E, int lmax, int C, int ps, int wm, int bad_index) {
  const int K = (lmax + 1) * (lmax + 1);
  const int P = oracle_paths(lmax, ps, NULL);
  const int NB = 8;
  const int64_t nw = wm ? (int64_t)NB * P * C : (int64_t)P * C;
  double* v = (double*)xmalloc(sizeof(double) * 3 * E);
  float* vf = (float*)xmalloc(sizeof(float) * 3 * E);
  int32_t* src = (int32_t*)xmalloc(sizeof(int32_t) * E);
  int32_t* dst = (int32_t*)xmalloc(sizeof(int32_t) * E);
  double* x = (double*)xmalloc(sizeof(double) * N * C * K);
  float* xf = (float*)xmalloc(sizeof(float) * N * C * K);
  double* w = (double*)xmalloc(sizeof(double) * nw);
  float* wf = (float*)xmalloc(sizeof(float) * nw);
  double* out = (double*)xmalloc(sizeof(double) * N * C * K);
  double* msg = (double*)xmalloc(sizeof(double) * E * C * K);
  fill_vectors(E, v);
  for (int64_t i = 0; i < 3 * E; ++i) vf[i] = (float)v[i];
  for (int64_t e = 0; e < E; ++e) {
    src[e] = N > 0 ? index_below(N) : 0;
    dst[e] = N > 0 ? index_below(N) : 0;
  }
  if (bad_index && E > 0) {
    src[E - 1] = (int32_t)N;
    dst[0] = -1;
  }
  for (int64_t i = 0; i < N * C * K; ++i) xf[i] = (float)(x[i] = uniform(-1.0, 1.0));
  for (int64_t i = 0; i < nw; ++i) wf[i] = (float)(w[i] = uniform(-1.0, 1.0));
  const int want = (bad_index && E > 0) ? 2 : 0;
  EXPECT(oracle_conv_f64(N, E, lmax, C, ps, wm, 5.0, NB, v, src, dst, x, w, out) == want);
  EXPECT(oracle_conv(N, E, lmax, C, ps, wm, 5.0, NB, vf, src, dst, xf, wf, out) == want);
  EXPECT(oracle_messages_f64(N, E, lmax, C, ps, wm, 5.0, NB, v, src, x, w, msg) == want);
  EXPECT(oracle_messages(N, E, lmax, C, ps, wm, 5.0, NB, vf, src, xf, wf, msg) == want);
  {
    /* radial-weight gradients (their own weights [8, P*C]), every subset of outputs */
    const int64_t nr = (int64_t)NB * P * C;
    double* Wr = (double*)xmalloc(sizeof(double) * nr);
    float* Wrf = (float*)xmalloc(sizeof(float) * nr);
    double* gout = (double*)xmalloc(sizeof(double) * N * C * K);
    float* goutf = (float*)xmalloc(sizeof(float) * N * C * K);
    double* gx = (double*)xmalloc(sizeof(double) * N * C * K);
    double* gW = (double*)xmalloc(sizeof(double) * nr);
    double* gvec = (double*)xmalloc(sizeof(double) * 3 * E);
    for (int64_t i = 0; i < nr; ++i) Wrf[i] = (float)(Wr[i] = uniform(-1.0, 1.0));
    for (int64_t i = 0; i < N * C * K; ++i) goutf[i] = (float)(gout[i] = uniform(-1.0, 1.0));
    for (int mask = 0; mask < 8; ++mask)
      EXPECT(oracle_conv_backward_radial_f64(N, E, lmax, C, ps, 5.0, NB, v, src, dst, x, Wr, gout,
                                             (mask & 1) ? gx : NULL, (mask & 2) ? gW : NULL,
                                             (mask & 4) ? gvec : NULL) == want);
    EXPECT(oracle_conv_backward_radial(N, E, lmax, C, ps, 5.0, NB, vf, src, dst, xf, Wrf, goutf, gx, gW, gvec) ==
           want);
    free(Wr);
    free(Wrf);
    free(gout);
    free(goutf);
    free(gx);
    free(gW);
    free(gvec);
  }
  if (!wm) {
    double* gout = (double*)xmalloc(sizeof(double) * N * C * K);
    float* goutf = (float*)xmalloc(sizeof(float) * N * C * K);
    double* gx = (double*)xmalloc(sizeof(double) * N * C * K);
    double* gw = (double*)xmalloc(sizeof(double) * P * C);
    double* gvec = (double*)xmalloc(sizeof(double) * 3 * E);
    for (int64_t i = 0; i < N * C * K; ++i) goutf[i] = (float)(gout[i] = uniform(-1.0, 1.0));
    for (int mask = 0; mask < 8; ++mask)
      EXPECT(oracle_conv_backward_f64(N, E, lmax, C, ps, v, src, dst, x, w, gout, (mask & 1) ? gx : NULL,
                                      (mask & 2) ? gw : NULL, (mask & 4) ? gvec : NULL) == want);
    EXPECT(oracle_conv_backward(N, E, lmax, C, ps, vf, src, dst, xf, wf, goutf, gx, gw, gvec) == want);
    free(gout);
    free(goutf);
    free(gx);
    free(gw);
    free(gvec);
  }
  free(v);
  free(vf);
  free(src);
  free(dst);
  free(x);
  free(xf);
  free(w);
  free(wf);
  free(out);
  free(msg);
}

static void test_conv(void) {
  for (int lmax = 0; lmax <= 4; ++lmax)
    for (int ps = 0; ps <= 1; ++ps)
      for (int wm = 0; wm <= 1; ++wm) conv_case(7, 23, lmax, lmax <= 3 ? 3 : 1, ps, wm, 0);
  conv_case(4, 9, 6, 1, 0, 0, 0); /* the largest lmax of the GPU kernels */
  conv_case(0, 0, 2, 4, 0, 0, 0);  /* no nodes, no edges */
  conv_case(5, 0, 3, 2, 1, 1, 0);  /* nodes without edges */
  conv_case(1, 9, 3, 2, 0, 0, 0);  /* one node: every edge is a self loop */
  conv_case(6, 14, 3, 2, 0, 0, 1); /* out-of-range indices */
  conv_case(6, 14, 2, 2, 1, 1, 1);
  /* invalid arguments are refused before any buffer is touched */
  EXPECT(oracle_conv_f64(1, 0, 13, 1, 0, 0, 5.0, 8, NULL, NULL, NULL, NULL, NULL, NULL) == 1);
  EXPECT(oracle_conv_f64(1, 0, 2, 0, 0, 0, 5.0, 8, NULL, NULL, NULL, NULL, NULL, NULL) == 1);
  EXPECT(oracle_conv_f64(1, 0, 2, 1, 0, 2, 5.0, 8, NULL, NULL, NULL, NULL, NULL, NULL) == 1);
  EXPECT(oracle_conv_f64(1, 0, 2, 1, 0, 1, 0.0, 8, NULL, NULL, NULL, NULL, NULL, NULL) == 1);
  EXPECT(oracle_conv_f64(1, 0, 2, 1, 0, 1, 5.0, 65, NULL, NULL, NULL, NULL, NULL, NULL) == 1);
  EXPECT(oracle_conv(1, 0, 2, 1, 3, 0, 5.0, 8, NULL, NULL, NULL, NULL, NULL, NULL) == 1);
  EXPECT(oracle_messages(-1, 0, 2, 1, 0, 0, 5.0, 8, NULL, NULL, NULL, NULL, NULL) == 1);
  EXPECT(oracle_conv_backward(1, 0, 2, 1, 5, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == 1);
  EXPECT(oracle_conv_backward_radial_f64(1, 0, 2, 1, 0, 0.0, 8, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                                         NULL) == 1);
  EXPECT(oracle_conv_backward_radial(1, 0, 2, 1, 0, 5.0, 65, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL) ==
         1);
}

static void test_interaction(void) {
  const int H = 5, NB = 8;
  for (int lmax = 0; lmax <= 3; ++lmax) {
    const int64_t N = 6, E = 14;
    const int C = 2, K = (lmax + 1) * (lmax + 1), P = oracle_paths(lmax, 0, NULL);
    float* vec = (float*)xmalloc(sizeof(float) * 3 * E);
    double* vd = (double*)xmalloc(sizeof(double) * 3 * E);
    int32_t* src = (int32_t*)xmalloc(sizeof(int32_t) * E);
    int32_t* dst = (int32_t*)xmalloc(sizeof(int32_t) * E);
    float* h = (float*)xmalloc(sizeof(float) * N * C * K);
    float* wu = (float*)xmalloc(sizeof(float) * (lmax + 1) * C * C);
    float* wo = (float*)xmalloc(sizeof(float) * (lmax + 1) * C * C);
    float* w1 = (float*)xmalloc(sizeof(float) * NB * H);
    float* w2 = (float*)xmalloc(sizeof(float) * H * H);
    float* w3 = (float*)xmalloc(sizeof(float) * H * P * C);
    double* out = (double*)xmalloc(sizeof(double) * N * C * K);
    double* phi = (double*)xmalloc(sizeof(double) * E * H);
    double* w1d = (double*)xmalloc(sizeof(double) * NB * H);
    double* w2d = (double*)xmalloc(sizeof(double) * H * H);
    fill_vectors(E, vd);
    for (int64_t i = 0; i < 3 * E; ++i) vec[i] = (float)vd[i];
    for (int64_t e = 0; e < E; ++e) {
      src[e] = index_below(N);
      dst[e] = index_below(N);
    }
    for (int64_t i = 0; i < N * C * K; ++i) h[i] = (float)uniform(-1, 1);
    for (int64_t i = 0; i < (lmax + 1) * C * C; ++i) {
      wu[i] = (float)uniform(-1, 1);
      wo[i] = (float)uniform(-1, 1);
    }
    for (int64_t i = 0; i < NB * H; ++i) w1d[i] = w1[i] = (float)uniform(-1, 1);
    for (int64_t i = 0; i < H * H; ++i) w2d[i] = w2[i] = (float)uniform(-1, 1);
    for (int64_t i = 0; i < H * P * C; ++i) w3[i] = (float)uniform(-1, 1);
    EXPECT(oracle_interaction(N, E, lmax, C, 0, 5.0, NB, H, vec, src, dst, h, wu, w1, w2, w3, wo, 2.0, out) == 0);
    EXPECT(oracle_interaction(N, 0, lmax, C, 0, 5.0, NB, H, vec, src, dst, h, wu, w1, w2, w3, wo, 2.0, out) == 0);
    EXPECT(oracle_radial_mlp_f64(E, vd, 5.0, NB, H, w1d, w2d, phi) == 0);
    EXPECT(oracle_interaction(N, E, lmax, C, 0, 5.0, NB, H, vec, src, dst, h, wu, w1, w2, w3, wo, 0.0, out) == 1);
    free(vec);
    free(vd);
    free(src);
    free(dst);
    free(h);
    free(wu);
    free(wo);
    free(w1);
    free(w2);
    free(w3);
    free(out);
    free(phi);
    free(w1d);
    free(w2d);
  }
  EXPECT(oracle_silu(0.0) == 0.0);
  EXPECT(oracle_conv_basis_f64(1, 1, 2, 1, 0, 4, NULL, NULL, NULL, NULL, NULL, NULL, NULL) == 1);
}

static void test_linear(void) {
  for (int lmax = 0; lmax <= 6; ++lmax) {
    const int C = 5;
    const int64_t N = 3;
    const int K = (lmax + 1) * (lmax + 1);
    float* h = (float*)xmalloc(sizeof(float) * N * C * K);
    float* W = (float*)xmalloc(sizeof(float) * (lmax + 1) * C * C);
    double* hd = (double*)xmalloc(sizeof(double) * N * C * K);
    double* Wd = (double*)xmalloc(sizeof(double) * (lmax + 1) * C * C);
    double* out = (double*)xmalloc(sizeof(double) * N * C * K);
    for (int64_t i = 0; i < N * C * K; ++i) h[i] = (float)(hd[i] = uniform(-2.0, 2.0));
    for (int64_t i = 0; i < (int64_t)(lmax + 1) * C * C; ++i) W[i] = (float)(Wd[i] = uniform(-2.0, 2.0));
    EXPECT(oracle_linear(N, C, lmax, 0, h, W, out) == 0);
    EXPECT(oracle_linear(N, C, lmax, 1, h, W, out) == 0);
    EXPECT(oracle_linear_f64(N, C, lmax, hd, Wd, out) == 0);
    EXPECT(oracle_linear(0, C, lmax, 1, h, W, out) == 0);
    free(h);
    free(W);
    free(hd);
    free(Wd);
    free(out);
  }
  EXPECT(oracle_linear(1, 0, 2, 0, NULL, NULL, NULL) == 1);
  EXPECT(oracle_linear_f64(1, 2, 13, NULL, NULL, NULL) == 1);
  const float specials[] = {0.0f, -0.0f, 1.0f, -1.5f, 1e-40f, -1e-45f, 3.4028235e38f, INFINITY, -INFINITY, NAN};
  for (int i = 0; i < 10; ++i) {
    const float r = oracle_round_bf16(specials[i]);
    EXPECT(isnan(specials[i]) ? isnan(r) : 1);
  }
}

int main(void) {
  oracle_set_threads(1);
  EXPECT(oracle_num_threads() >= 1);
  test_sh();
  test_cg_and_paths();
  test_radial();
  test_conv();
  test_linear();
  test_interaction();
  /* the row-, edge- and node-parallel loops with several threads */
  oracle_set_threads(3);
  test_conv();
  test_linear();
  test_interaction();
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("oracle sanitizer run: all entry points clean\n");
  return 0;
}
