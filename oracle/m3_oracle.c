/*
 * m3_oracle.c -- plain, slow fp64 CPU reference of the Mamba-3 SSM layer
 * recurrence (prefill over a whole sequence, and one decode step).
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the parity oracle.  Only the
 * test suite, the smoke check and the benchmark's CPU-baseline leg may load
 * it.  It shares no source, header, table or helper with the GPU library, and
 * the GPU library never calls it.
 *
 * What it computes (one independent unit per (batch b, head h)):
 *
 *   The state is complex: N/2 complex rows z_k (k = 0..N/2-1), P columns.
 *   Real storage pairs rows (2k, 2k+1) as (Re z_k, Im z_k).  B_t and C_t
 *   (N x R, stored [R][N]) pair the same way: b_k = B[2k] + i B[2k+1].
 *
 *   Exponential-trapezoidal rule with a complex transition
 *   (Mamba-3 paper summary, aipaper.cc, "Mathematical formulas", Proposition 1;
 *   Mamba-3 explainer, yunpan.plus, "first improvement: exponential-trapezoidal
 *   discretisation" and "second improvement: complex-valued state space"):
 *
 *     alpha_t = exp(dt_t * (A + i*theta_t[k]))             (complex, per pair)
 *     beta_t  = (1 - lam_t) * dt_t * alpha_t
 *     gamma_t = lam_t * dt_t
 *     z_t     = alpha_t z_{t-1} + beta_t (b_{t-1} x_{t-1}^T) + gamma_t (b_t x_t^T)
 *     y_t[r]  = sum_k Re(conj(c_k[r]) z_t[k])  ==  C_t^T h_t  in real storage
 *
 *   The per-pair factor exp(i dt theta) is the 2x2 rotation
 *   [[cos, -sin], [sin, cos]] acting on (Re, Im) (explainer, block-diagonal
 *   rotation matrices).  MIMO: x_t is P x R and B_t, C_t are N x R, so
 *   b x^T is the rank-R sum over r (paper summary, item 3; explainer, third
 *   improvement).  dt, lam, theta and A are shared by the R ranks.
 *
 *   Start of a sequence: z_{-1} = h0 (zero if not given) and the previous
 *   input term b_{-1} x_{-1}^T is the given halo (zero if not given).
 *
 * Layouts (row-major, dense):
 *   x [B,T,H,R,P]; B, C [B,T,H,R,N]; dt, lam [B,T,H]; theta [B,T,H,N/2];
 *   A [H]; y [B,T,H,R,P]; h0, h_final [B,H,N,P].
 * Inputs are float (the exact values the GPU path sees); arithmetic and
 * outputs are double.
 */
#include <complex.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define M3O_OK 0
#define M3O_EINVAL 1
#define M3O_ENOMEM 2

typedef struct {
  int64_t nb, nt, nh, np, nn, nr; /* batch, seqlen, heads, P, N, R */
} dims_t;

/* One step of the recurrence for one (b,h) unit.  z: [N/2][P] complex state,
 * updated in place.  prev_b/prev_x may be NULL (no previous input term).
 * Bt [R][N], xt [R][P], th [N/2].  If Ct != NULL, writes y [R][P]. */
static void one_step(double complex *z, int64_t nn, int64_t np, int64_t nr,
                     double dt, double a, double lam, const float *th,
                     const float *prev_b, const float *prev_x,
                     const float *Bt, const float *xt, const float *Ct,
                     double *y) {
  const int64_t npair = nn / 2;
  const double gamma = lam * dt;
  for (int64_t k = 0; k < npair; ++k) {
    const double complex alpha = cexp(dt * (a + I * (double)th[k]));
    const double complex beta = (1.0 - lam) * dt * alpha;
    for (int64_t p = 0; p < np; ++p) {
      double complex bx_prev = 0.0, bx_cur = 0.0;
      for (int64_t r = 0; r < nr; ++r) {
        if (prev_b) {
          const double complex bk =
              (double)prev_b[r * nn + 2 * k] + I * (double)prev_b[r * nn + 2 * k + 1];
          bx_prev += bk * (double)prev_x[r * np + p];
        }
        const double complex bk =
            (double)Bt[r * nn + 2 * k] + I * (double)Bt[r * nn + 2 * k + 1];
        bx_cur += bk * (double)xt[r * np + p];
      }
      z[k * np + p] = alpha * z[k * np + p] + beta * bx_prev + gamma * bx_cur;
    }
  }
  if (Ct && y) {
    for (int64_t r = 0; r < nr; ++r) {
      for (int64_t p = 0; p < np; ++p) {
        double acc = 0.0;
        for (int64_t k = 0; k < npair; ++k) {
          const double complex ck =
              (double)Ct[r * nn + 2 * k] + I * (double)Ct[r * nn + 2 * k + 1];
          acc += creal(conj(ck) * z[k * np + p]);
        }
        y[r * np + p] = acc;
      }
    }
  }
}

static void load_state(double complex *z, const double *h, int64_t nn, int64_t np) {
  for (int64_t k = 0; k < nn / 2; ++k)
    for (int64_t p = 0; p < np; ++p)
      z[k * np + p] = h[(2 * k) * np + p] + I * h[(2 * k + 1) * np + p];
}

static void store_state(const double complex *z, double *h, int64_t nn, int64_t np) {
  for (int64_t k = 0; k < nn / 2; ++k)
    for (int64_t p = 0; p < np; ++p) {
      h[(2 * k) * np + p] = creal(z[k * np + p]);
      h[(2 * k + 1) * np + p] = cimag(z[k * np + p]);
    }
}

/* ------------------------------------------------------------------------ */
/* prefill                                                                   */

typedef struct {
  dims_t d;
  const float *x, *dt, *A, *lam, *theta, *B, *C, *x_halo, *B_halo;
  const double *h0;
  double *y, *h_final;
  const int64_t *units;
  int64_t n_units;
  int tid, nthreads, status;
} prefill_job;

static void prefill_unit(const prefill_job *j, int64_t unit, double complex *z) {
  const dims_t d = j->d;
  const int64_t b = unit / d.nh, h = unit % d.nh;
  const int64_t nn = d.nn, np = d.np, nr = d.nr, npair = nn / 2;
  if (j->h0)
    load_state(z, j->h0 + unit * nn * np, nn, np);
  else
    memset(z, 0, sizeof(double complex) * (size_t)(npair * np));
  const float *prev_b = j->B_halo ? j->B_halo + unit * nr * nn : NULL;
  const float *prev_x = j->x_halo ? j->x_halo + unit * nr * np : NULL;
  if (!prev_b || !prev_x) prev_b = prev_x = NULL;
  for (int64_t t = 0; t < d.nt; ++t) {
    const int64_t bth = (b * d.nt + t) * d.nh + h; /* index into [B,T,H] */
    const float *Bt = j->B + bth * nr * nn;
    const float *Ct = j->C + bth * nr * nn;
    const float *xt = j->x + bth * nr * np;
    double *yt = j->y ? j->y + bth * nr * np : NULL;
    one_step(z, nn, np, nr, (double)j->dt[bth], (double)j->A[h], (double)j->lam[bth],
             j->theta + bth * npair, prev_b, prev_x, Bt, xt, Ct, yt);
    prev_b = Bt;
    prev_x = xt;
  }
  if (j->h_final) store_state(z, j->h_final + unit * nn * np, nn, np);
}

static void *prefill_worker(void *arg) {
  prefill_job *j = (prefill_job *)arg;
  double complex *z = malloc(sizeof(double complex) * (size_t)(j->d.nn / 2 * j->d.np));
  if (!z) {
    j->status = M3O_ENOMEM;
    return NULL;
  }
  for (int64_t i = j->tid; i < j->n_units; i += j->nthreads)
    prefill_unit(j, j->units ? j->units[i] : i, z);
  free(z);
  return NULL;
}

static int resolve_threads(int nthreads, int64_t n_units) {
  if (nthreads <= 0) {
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    nthreads = n > 0 ? (int)n : 1;
  }
  if (nthreads > n_units) nthreads = (int)(n_units > 0 ? n_units : 1);
  if (nthreads > 256) nthreads = 256;
  return nthreads;
}

/* Returns 0 on success.  units: optional list of unit ids (b*H + h) to compute;
 * NULL means all B*H units.  Outputs of units not listed are left untouched. */
int m3o_prefill(const int64_t dims6[6], const float *x, const float *dt, const float *A,
                const float *lam, const float *theta, const float *B, const float *C,
                const double *h0, const float *x_halo, const float *B_halo, double *y,
                double *h_final, const int64_t *units, int64_t n_units, int nthreads) {
  if (!dims6 || !x || !dt || !A || !lam || !theta || !B || !C) return M3O_EINVAL;
  dims_t d = {dims6[0], dims6[1], dims6[2], dims6[3], dims6[4], dims6[5]};
  if (d.nb < 0 || d.nt < 0 || d.nh < 1 || d.np < 1 || d.nn < 2 || d.nn % 2 || d.nr < 1)
    return M3O_EINVAL;
  if (!units) n_units = d.nb * d.nh;
  for (int64_t i = 0; units && i < n_units; ++i)
    if (units[i] < 0 || units[i] >= d.nb * d.nh) return M3O_EINVAL;
  if (n_units == 0) return M3O_OK;
  int nt = resolve_threads(nthreads, n_units);
  prefill_job *jobs = calloc((size_t)nt, sizeof(prefill_job));
  pthread_t *th = calloc((size_t)nt, sizeof(pthread_t));
  if (!jobs || !th) {
    free(jobs);
    free(th);
    return M3O_ENOMEM;
  }
  int status = M3O_OK;
  for (int i = 0; i < nt; ++i) {
    prefill_job j = {d, x, dt, A, lam, theta, B, C, x_halo, B_halo, h0,
                     y, h_final, units, n_units, i, nt, M3O_OK};
    jobs[i] = j;
    if (pthread_create(&th[i], NULL, prefill_worker, &jobs[i]) != 0) {
      prefill_worker(&jobs[i]); /* run inline if a thread cannot start */
      th[i] = 0;
    }
  }
  for (int i = 0; i < nt; ++i) {
    if (th[i]) pthread_join(th[i], NULL);
    if (jobs[i].status != M3O_OK) status = jobs[i].status;
  }
  free(jobs);
  free(th);
  return status;
}

/* ------------------------------------------------------------------------ */
/* decode step                                                               */

typedef struct {
  dims_t d; /* nb = number of sequences S; nt unused */
  const double *h_in;
  const float *x_t, *x_prev, *B_t, *B_prev, *C_t, *dt, *A, *lam, *theta;
  double *y, *h_out;
  const int64_t *units;
  int64_t n_units;
  int tid, nthreads, status;
} decode_job;

static void *decode_worker(void *arg) {
  decode_job *j = (decode_job *)arg;
  const dims_t d = j->d;
  const int64_t nn = d.nn, np = d.np, nr = d.nr, npair = nn / 2;
  double complex *z = malloc(sizeof(double complex) * (size_t)(npair * np));
  if (!z) {
    j->status = M3O_ENOMEM;
    return NULL;
  }
  for (int64_t i = j->tid; i < j->n_units; i += j->nthreads) {
    const int64_t unit = j->units ? j->units[i] : i; /* = s*H + h */
    const int64_t h = unit % d.nh;
    load_state(z, j->h_in + unit * nn * np, nn, np);
    one_step(z, nn, np, nr, (double)j->dt[unit], (double)j->A[h], (double)j->lam[unit],
             j->theta + unit * npair, j->B_prev + unit * nr * nn, j->x_prev + unit * nr * np,
             j->B_t + unit * nr * nn, j->x_t + unit * nr * np, j->C_t + unit * nr * nn,
             j->y + unit * nr * np);
    store_state(z, j->h_out + unit * nn * np, nn, np);
  }
  free(z);
  return NULL;
}

/* One decode step for S sequences.  dims6 = {S, (ignored), H, P, N, R}.
 * Layouts: h_in, h_out [S,H,N,P] (may alias); x_t, x_prev, y [S,H,R,P];
 * B_t, B_prev, C_t [S,H,R,N]; dt, lam [S,H]; theta [S,H,N/2]; A [H]. */
int m3o_decode_step(const int64_t dims6[6], const double *h_in, const float *x_t,
                    const float *x_prev, const float *B_t, const float *B_prev,
                    const float *C_t, const float *dt, const float *A, const float *lam,
                    const float *theta, double *y, double *h_out, const int64_t *units,
                    int64_t n_units, int nthreads) {
  if (!dims6 || !h_in || !x_t || !x_prev || !B_t || !B_prev || !C_t || !dt || !A || !lam ||
      !theta || !y || !h_out)
    return M3O_EINVAL;
  dims_t d = {dims6[0], dims6[1], dims6[2], dims6[3], dims6[4], dims6[5]};
  if (d.nb < 0 || d.nh < 1 || d.np < 1 || d.nn < 2 || d.nn % 2 || d.nr < 1) return M3O_EINVAL;
  if (!units) n_units = d.nb * d.nh;
  for (int64_t i = 0; units && i < n_units; ++i)
    if (units[i] < 0 || units[i] >= d.nb * d.nh) return M3O_EINVAL;
  if (n_units == 0) return M3O_OK;
  int nt = resolve_threads(nthreads, n_units);
  decode_job *jobs = calloc((size_t)nt, sizeof(decode_job));
  pthread_t *th = calloc((size_t)nt, sizeof(pthread_t));
  if (!jobs || !th) {
    free(jobs);
    free(th);
    return M3O_ENOMEM;
  }
  int status = M3O_OK;
  for (int i = 0; i < nt; ++i) {
    decode_job j = {d, h_in, x_t, x_prev, B_t, B_prev, C_t, dt, A, lam, theta,
                    y, h_out, units, n_units, i, nt, M3O_OK};
    jobs[i] = j;
    if (pthread_create(&th[i], NULL, decode_worker, &jobs[i]) != 0) {
      decode_worker(&jobs[i]);
      th[i] = 0;
    }
  }
  for (int i = 0; i < nt; ++i) {
    if (th[i]) pthread_join(th[i], NULL);
    if (jobs[i].status != M3O_OK) status = jobs[i].status;
  }
  free(jobs);
  free(th);
  return status;
}

int m3o_version(void) { return 1; }
