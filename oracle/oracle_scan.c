/*
 * fp64 CPU oracle for the S6 selective scan -- TEST INFRASTRUCTURE ONLY.
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may load or call this code.  It shares no
 * code, header, table or helper with the HIP library; it is the plain sequential definition, written out.
 *
 * What it computes (sources: the Mamba paper, arXiv 2312.00752, as translated on gitcode.csdn.net, sections 2 and
 * 3.2-3.6; the ifdog.com Mamba tutorial, sections "连续状态空间模型", "离散化" and "Mamba：选择性状态空间模型"):
 *   per batch b, channel d (the SSM runs on every channel independently, paper section 2 "structure and dimensions"):
 *     h[n] = h0[b,d,n] (0 when h0 is absent)
 *     for t = 0 .. L-1:
 *       u     = dt[b,d,t] + dt_bias[d]
 *       Delta = softplus(u) = log(1 + e^u)          (paper section 3.2: tau_Delta = softplus; tutorial: softplus def.)
 *               or u itself when softplus is off
 *       for n: abar = exp(Delta * A[d,n])             (ZOH for A; tutorial "离散化", diagonal case)
 *              bbar = Delta * B[b,n,t]                (Euler rule for B, the tutorial's simplified selective toy)
 *                  or expm1(Delta*A)/A * B[b,n,t]     (ZOH for B, paper eq. (4) as written out in the tutorial;
 *                                                      A == 0 takes the limit Delta * B)
 *              h[n]  = abar * h[n] + bbar * x[b,d,t]  (linear recurrence (2))
 *       y = sum_n C[b,n,t] * h[n] + Dskip[d] * x[b,d,t]   (output equation y = Ch + Dx, tutorial)
 *       y = y * z * sigmoid(z)  when the gate z is given  (Mamba block: SSM branch times SiLU of the gate branch)
 *     h_final[b,d,:] = h
 *   The single-token decode step (constant time per step, paper section 1 (ii)) is the same body for one t, with the
 *   state read from and written back to the caller's array.
 *
 * Layouts (all row-major, fp64): x, dt, z, y: [batch][dim][seqlen]; B, C: [batch][dstate][seqlen]; A: [dim][dstate];
 * dt_bias, Dskip: [dim]; h0, h_final, decode state: [batch][dim][dstate].  Optional pointers may be NULL.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* softplus(u) = log(1 + e^u), evaluated as max(u, 0) + log1p(exp(-|u|)) so that it is accurate at both ends. */
static double sp(double u) { return u > 0.0 ? u + log1p(exp(-u)) : log1p(exp(u)); }

/* One time step for one channel: updates h[0..N-1] and returns the gated output. */
static double step(int64_t N, int disc, int use_softplus, double xv, double dtv, double bias, const double* A_row,
                   const double* Bt, int64_t Bstride, const double* Ct, int64_t Cstride, int has_D, double Dv,
                   int has_z, double zv, double* h) {
  double u = dtv + bias;
  double delta = use_softplus ? sp(u) : u;
  double y = 0.0;
  for (int64_t n = 0; n < N; n++) {
    double An = A_row[n];
    double abar = exp(delta * An);
    double coef;
    if (disc == 0) {
      coef = delta;
    } else {
      coef = (An == 0.0) ? delta : expm1(delta * An) / An;
    }
    h[n] = abar * h[n] + coef * Bt[n * Bstride] * xv;
    y += Ct[n * Cstride] * h[n];
  }
  if (has_D) y += Dv * xv;
  if (has_z) y *= zv / (1.0 + exp(-zv));
  return y;
}

int oracle_scan_f64(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int disc, int use_softplus,
                    const double* x, const double* dt, const double* dt_bias, const double* A, const double* B,
                    const double* C, const double* Dskip, const double* z, const double* h0, double* y,
                    double* h_final, int nthreads) {
  if (batch < 0 || dim < 0 || seqlen < 0 || dstate < 1 || dstate > 4096) return 1;
  if (!x || !dt || !A || !B || !C || !y) return 2;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  int64_t nch = batch * dim;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t ch = 0; ch < nch; ch++) {
    int64_t b = ch / dim, d = ch % dim;
    double h[4096];
    for (int64_t n = 0; n < dstate; n++) h[n] = h0 ? h0[ch * dstate + n] : 0.0;
    const double* xr = x + ch * seqlen;
    const double* dr = dt + ch * seqlen;
    const double* zr = z ? z + ch * seqlen : NULL;
    double* yr = y + ch * seqlen;
    const double* Bb = B + b * dstate * seqlen;
    const double* Cb = C + b * dstate * seqlen;
    double bias = dt_bias ? dt_bias[d] : 0.0;
    double Dv = Dskip ? Dskip[d] : 0.0;
    for (int64_t t = 0; t < seqlen; t++) {
      yr[t] = step(dstate, disc, use_softplus, xr[t], dr[t], bias, A + d * dstate, Bb + t, seqlen, Cb + t, seqlen,
                   Dskip != NULL, Dv, zr != NULL, zr ? zr[t] : 0.0, h);
    }
    if (h_final)
      for (int64_t n = 0; n < dstate; n++) h_final[ch * dstate + n] = h[n];
  }
  return 0;
}

int oracle_state_update_f64(int64_t batch, int64_t dim, int64_t dstate, int disc, int use_softplus, double* state,
                            const double* x, const double* dt, const double* dt_bias, const double* A,
                            const double* B, const double* C, const double* Dskip, const double* z, double* y,
                            int nthreads) {
  if (batch < 0 || dim < 0 || dstate < 1 || dstate > 4096) return 1;
  if (!state || !x || !dt || !A || !B || !C || !y) return 2;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  int64_t nch = batch * dim;
#pragma omp parallel for schedule(static)
  for (int64_t ch = 0; ch < nch; ch++) {
    int64_t b = ch / dim, d = ch % dim;
    y[ch] = step(dstate, disc, use_softplus, x[ch], dt[ch], dt_bias ? dt_bias[d] : 0.0, A + d * dstate,
                 B + b * dstate, 1, C + b * dstate, 1, Dskip != NULL, Dskip ? Dskip[d] : 0.0, z != NULL,
                 z ? z[ch] : 0.0, state + ch * dstate);
  }
  return 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
