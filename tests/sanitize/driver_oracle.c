/* Host driver of the fp64 oracle (oracle/m3_oracle.c) for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer: prefill over a few
 * shapes (with and without a unit subset, an initial state and a halo) and
 * decode steps, on inputs from a fixed linear congruential generator.
 * Checks that every output is finite and that a unit subset reproduces the
 * full run's units bit for bit.  Exit status 0 when every check holds. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int m3o_prefill(const int64_t dims6[6], const float* x, const float* dt, const float* A,
                const float* lam, const float* theta, const float* B, const float* C,
                const double* h0, const float* x_halo, const float* B_halo, double* y,
                double* h_final, const int64_t* units, int64_t n_units, int nthreads);
int m3o_decode_step(const int64_t dims6[6], const double* h_in, const float* x_t,
                    const float* x_prev, const float* B_t, const float* B_prev, const float* C_t,
                    const float* dt, const float* A, const float* lam, const float* theta,
                    double* y, double* h_out, const int64_t* units, int64_t n_units,
                    int nthreads);

static uint64_t state = 88172645463325252ull;
static double uniform(void) { /* [0, 1) */
  state = state * 6364136223846793005ull + 1442695040888963407ull;
  return (double)(state >> 11) * (1.0 / 9007199254740992.0);
}
static float* fill(size_t n, double lo, double hi) {
  float* a = malloc((n ? n : 1) * sizeof(float));
  for (size_t i = 0; i < n; ++i) a[i] = (float)(lo + (hi - lo) * uniform());
  return a;
}
static int all_finite(const double* a, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(a[i])) return 0;
  return 1;
}

static int fails = 0;

static void one_shape(int64_t nb, int64_t nt, int64_t nh, int64_t np, int64_t nn, int64_t nr,
                      int with_state) {
  const int64_t dims[6] = {nb, nt, nh, np, nn, nr};
  const size_t tok = (size_t)nb * nt * nh;
  float* x = fill(tok * nr * np, -1, 1);
  float* dt = fill(tok, 0.05, 1.0);
  float* A = fill(nh, -2, -0.1);
  float* lam = fill(tok, 0, 1);
  float* th = fill(tok * nn / 2, -3.14, 3.14);
  float* B = fill(tok * nr * nn, -0.3, 0.3);
  float* C = fill(tok * nr * nn, -0.3, 0.3);
  const size_t hs = (size_t)nb * nh * nn * np;
  double* h0 = NULL;
  float *xh = NULL, *bh = NULL;
  if (with_state) {
    h0 = malloc(hs * sizeof(double));
    for (size_t i = 0; i < hs; ++i) h0[i] = uniform() - 0.5;
    xh = fill((size_t)nb * nh * nr * np, -1, 1);
    bh = fill((size_t)nb * nh * nr * nn, -0.3, 0.3);
  }
  const size_t ys = tok * nr * np;
  double* y = malloc((ys ? ys : 1) * sizeof(double));
  double* hf = malloc(hs * sizeof(double));
  double* y2 = malloc((ys ? ys : 1) * sizeof(double));
  double* hf2 = malloc(hs * sizeof(double));
  if (m3o_prefill(dims, x, dt, A, lam, th, B, C, h0, xh, bh, y, hf, NULL, 0, 3) != 0) ++fails;
  if (!all_finite(y, ys) || !all_finite(hf, hs)) ++fails;
  /* the last unit alone reproduces the full run's last unit bit for bit */
  const int64_t last = nb * nh - 1;
  for (size_t i = 0; i < ys; ++i) y2[i] = NAN;
  if (m3o_prefill(dims, x, dt, A, lam, th, B, C, h0, xh, bh, y2, hf2, &last, 1, 1) != 0) ++fails;
  const int64_t b = last / nh, h = last % nh;
  for (int64_t t = 0; t < nt; ++t)
    for (int64_t k = 0; k < nr * np; ++k) {
      const size_t i = ((size_t)(b * nt + t) * nh + h) * nr * np + k;
      if (memcmp(&y[i], &y2[i], sizeof(double)) != 0) ++fails;
    }
  /* decode steps from the final state, full batch */
  const int64_t ddims[6] = {nb, 1, nh, np, nn, nr};
  const size_t su = (size_t)nb * nh;
  double* yd = malloc(su * nr * np * sizeof(double));
  double* hn = malloc(hs * sizeof(double));
  for (int step = 0; step < 3; ++step) {
    if (m3o_decode_step(ddims, hf, x, x, B, B, C, dt, A, lam, th, yd, hn, NULL, 0, 2) != 0) ++fails;
    if (!all_finite(yd, su * nr * np) || !all_finite(hn, hs)) ++fails;
    memcpy(hf, hn, hs * sizeof(double));
  }
  free(x); free(dt); free(A); free(lam); free(th); free(B); free(C);
  free(h0); free(xh); free(bh); free(y); free(hf); free(y2); free(hf2); free(yd); free(hn);
}

int main(void) {
  one_shape(1, 37, 1, 16, 16, 1, 0);
  one_shape(2, 20, 3, 8, 6, 2, 1);
  one_shape(1, 5, 2, 4, 4, 4, 1);
  one_shape(3, 1, 1, 2, 2, 1, 0);
  /* rejected arguments */
  const int64_t bad[6] = {1, 4, 1, 4, 3, 1}; /* odd N */
  float f[64] = {0};
  if (m3o_prefill(bad, f, f, f, f, f, f, f, NULL, NULL, NULL, NULL, NULL, NULL, 0, 1) == 0) ++fails;
  const int64_t ok[6] = {1, 4, 1, 4, 4, 1};
  const int64_t out_of_range = 5;
  double yy[64], hh[64];
  if (m3o_prefill(ok, f, f, f, f, f, f, f, NULL, NULL, NULL, yy, hh, &out_of_range, 1, 1) == 0)
    ++fails;
  printf("driver_oracle: %d failures\n", fails);
  return fails ? 1 : 0;
}
