/*
 * ssm_oracle.c -- fp64 CPU reference of the selective state-space causal scan.
 *
 * TEST INFRASTRUCTURE ONLY (see ssm_oracle.h).  Plain, sequential per
 * channel, libm exp/log1p, no fast-math, no blocking or reordering: token t
 * of channel (b, c) is processed after token t-1, exactly as the recurrence
 * is written.  Threads only split the set of independent channels.
 *
 * Per channel (b, c), with xi the raw input x[b, c, :] and history
 * xi[-3..-1] taken from conv0 (or zero), h from h0 (or zero):
 *   v_t   = conv_b[c] + sum_{k=0..3} conv_w[c, k] * xi[t-3+k]     (causal conv)
 *   u_t   = v_t * sigmoid(v_t)                                     (SiLU)
 *   s_t   = dt[b, c, t] + dt_bias[c]
 *   D_t   = softplus(s_t) = max(s_t, 0) + log1p(exp(-|s_t|))      (step size)
 *   for n : h[n] = exp(D_t * A[c, n]) * h[n] + D_t * B[b, t, n] * u_t
 *   r_t   = sum_n C[b, t, n] * h[n] + Dskip[c] * u_t                (readout)
 *   y_t   = z ? r_t * z_t * sigmoid(z_t) : r_t                    (gate)
 * Afterwards h_out = h and conv_out[j] = xi[L-3+j], j = 0, 1, 2.
 *
 * Passages followed: "Scaling State-Space Models on Multiple GPUs with
 * Tensor Parallelism" (euno.news summary of arXiv 2602.21144), Methodology
 * item 2 (channel-local recurrence, state slice kept per GPU) and item 3
 * (the state left by prefill is cached and decode resumes from it); the
 * Key contributions list (state caching between prefill and decode).  The
 * update form is the standard Mamba selective scan (Gu & Dao, 2023).
 */
#include "ssm_oracle.h"
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int64_t B, L, D, N;
  const double *x, *dt, *z, *Bm, *Cm, *A, *Dskip, *dt_bias, *conv_w, *conv_b, *h0, *conv0;
  double *y, *h_out, *conv_out;
  int64_t first, last; /* channel range [first, last) over flattened (b, c) */
} job_t;

static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

static double softplus(double s) { return (s > 0.0 ? s : 0.0) + log1p(exp(-fabs(s))); }

static void scan_one_channel(const job_t* j, int64_t b, int64_t c, double* h) {
  const int64_t L = j->L, D = j->D, N = j->N;
  const int64_t row = b * D + c;                 /* (b, c) row of the [B, D, *] tensors */
  const double* xr = j->x + row * L;
  const double* dtr = j->dt + row * L;
  const double* zr = j->z ? j->z + row * L : NULL;
  double* yr = j->y + row * L;
  const double* w = j->conv_w + c * SSM_ORACLE_CONV_W;
  const double bias = j->conv_b ? j->conv_b[c] : 0.0;

  /* hist[0..2] = xi[t-3], xi[t-2], xi[t-1] (raw inputs, oldest first) */
  double hist[3] = {0.0, 0.0, 0.0};
  if (j->conv0) memcpy(hist, j->conv0 + row * 3, sizeof hist);
  for (int64_t n = 0; n < N; ++n) h[n] = j->h0 ? j->h0[row * N + n] : 0.0;

  for (int64_t t = 0; t < L; ++t) {
    const double xt = xr[t];
    const double v = bias + w[0] * hist[0] + w[1] * hist[1] + w[2] * hist[2] + w[3] * xt;
    const double u = v * sigmoid(v);
    const double delta = softplus(dtr[t] + j->dt_bias[c]);
    const double* Bt = j->Bm + (b * L + t) * N;
    const double* Ct = j->Cm + (b * L + t) * N;
    double r = 0.0;
    for (int64_t n = 0; n < N; ++n) {
      const double a = exp(delta * j->A[c * N + n]);
      h[n] = a * h[n] + delta * Bt[n] * u;
      r += Ct[n] * h[n];
    }
    r += j->Dskip[c] * u;
    yr[t] = zr ? r * zr[t] * sigmoid(zr[t]) : r;
    hist[0] = hist[1];
    hist[1] = hist[2];
    hist[2] = xt;
  }
  for (int64_t n = 0; n < N; ++n) j->h_out[row * N + n] = h[n];
  memcpy(j->conv_out + row * 3, hist, sizeof hist);
}

static void* run_job(void* arg) {
  const job_t* j = (const job_t*)arg;
  double* h = (double*)malloc((size_t)j->N * sizeof(double));
  if (!h) return (void*)1;
  for (int64_t r = j->first; r < j->last; ++r) scan_one_channel(j, r / j->D, r % j->D, h);
  free(h);
  return NULL;
}

int ssm_oracle_scan(int64_t B, int64_t L, int64_t D, int64_t N,
                    const double* x, const double* dt, const double* z,
                    const double* Bm, const double* Cm,
                    const double* A, const double* Dskip, const double* dt_bias,
                    const double* conv_w, const double* conv_b,
                    const double* h0, const double* conv0,
                    double* y, double* h_out, double* conv_out,
                    int nthreads) {
  if (B < 1 || L < 1 || D < 1 || N < 1) return -1;
  if (!x || !dt || !Bm || !Cm || !A || !Dskip || !dt_bias || !conv_w || !y || !h_out || !conv_out)
    return -1;
  job_t base = {B, L, D, N, x, dt, z, Bm, Cm, A, Dskip, dt_bias, conv_w, conv_b, h0, conv0,
                y, h_out, conv_out, 0, B * D};
  const int64_t rows = B * D;
  int64_t nt = nthreads < 1 ? 1 : nthreads;
  if (nt > rows) nt = rows;
  if (nt == 1) return run_job(&base) ? -1 : 0;

  pthread_t* tid = (pthread_t*)malloc((size_t)nt * sizeof(pthread_t));
  job_t* jobs = (job_t*)malloc((size_t)nt * sizeof(job_t));
  if (!tid || !jobs) { free(tid); free(jobs); return -1; }
  for (int64_t i = 0; i < nt; ++i) {
    jobs[i] = base;
    jobs[i].first = rows * i / nt;
    jobs[i].last = rows * (i + 1) / nt;
  }
  int rc = 0;
  int64_t started = 0;
  for (; started < nt; ++started)
    if (pthread_create(&tid[started], NULL, run_job, &jobs[started]) != 0) break;
  for (int64_t i = started; i < nt; ++i) /* threads unavailable: run the rest here */
    if (run_job(&jobs[i])) rc = -1;
  for (int64_t i = 0; i < started; ++i) {
    void* ret = NULL;
    pthread_join(tid[i], &ret);
    if (ret) rc = -1;
  }
  free(tid);
  free(jobs);
  return rc;
}
