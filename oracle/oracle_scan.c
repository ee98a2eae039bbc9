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
#include <stdlib.h>

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

/*
 * Backward of the scan (gradients of a scalar loss given dL/dy and optionally dL/dh_final), fp64.
 * The training path needs these gradients (Mamba paper, section 3.3.2, the recomputation paragraph: the backward pass
 * of the fused layer rebuilds the states from the inputs; alishangtian.com close reading, "hardware-aware algorithm",
 * item on recomputation).  They are the chain rule through the forward definition above, nothing more.
 * Recomputation is not needed here: the oracle keeps every state h_t of a channel.  Per channel, walking t from
 * L-1 down to 0 with the adjoint g = dL/dh_t:
 *   s_t = sum_n C h_t + D x_t (pre-gate output),  ds = dy * silu(z) (dy without gate),  dz = dy * s * silu'(z)
 *   g  += C_t * ds;  then with a = exp(Delta A), b-coefficient coef (Delta for Euler-B, expm1(Delta A)/A for ZOH):
 *   dDelta += g (d coef/dDelta B x + h_{t-1} a A),  dx += g coef B,  dB += g coef x,  dC += ds h_t,
 *   dA += g (d coef/dA B x + h_{t-1} a Delta),  g *= a  (adjoint of h_{t-1});   dx += ds D,  dD += ds x,
 *   du = dDelta * sigmoid(u) (softplus derivative; 1 when softplus is off),  ddt = du,  dbias += du,
 *   finally dh0 = g.
 * Layouts as the forward; dB, dC [b][N][L] (summed over channels), dA [D][N], dD, dbias [D] (summed over b, t).
 * Work is split over batch elements (each thread owns its batch's dB / dC); per-channel parameter gradients are
 * accumulated per batch element and summed afterwards in a fixed order, so results do not depend on threads.
 */
static double sigm(double v) { return 1.0 / (1.0 + exp(-v)); }

int oracle_scan_bwd_f64(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int disc, int use_softplus,
                        const double* x, const double* dt, const double* dt_bias, const double* A, const double* B,
                        const double* C, const double* Dskip, const double* z, const double* h0, const double* dy,
                        const double* dh_final, double* dx, double* ddt, double* ddt_bias, double* dA, double* dB,
                        double* dC, double* dD, double* dz, double* dh0, int nthreads) {
  if (batch < 0 || dim < 0 || seqlen < 1 || dstate < 1 || dstate > 4096) return 1;
  if (!x || !dt || !A || !B || !C || !dy || !dx || !ddt || !dA || !dB || !dC) return 2;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  const int64_t N = dstate, L = seqlen;
  /* per-batch partials of the per-channel parameter gradients */
  double* pA = (double*)calloc((size_t)(batch * dim * N), sizeof(double));
  double* pD = (double*)calloc((size_t)(batch * dim), sizeof(double));
  double* pb = (double*)calloc((size_t)(batch * dim), sizeof(double));
  if (!pA || !pD || !pb) {
    free(pA); free(pD); free(pb);
    return 3;
  }
  int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t b = 0; b < batch; b++) {
    double* H = (double*)malloc((size_t)((L + 1) * N) * sizeof(double)); /* H[t+1] = h_t, H[0] = h0 */
    double* Dl = (double*)malloc((size_t)L * sizeof(double));
    double* S = (double*)malloc((size_t)L * sizeof(double));
    double* g = (double*)malloc((size_t)N * sizeof(double));
    if (!H || !Dl || !S || !g) {
#pragma omp atomic write
      failed = 1;
      free(H); free(Dl); free(S); free(g);
      continue;
    }
    for (int64_t i = 0; i < N * L; i++) {
      dB[b * N * L + i] = 0.0;
      dC[b * N * L + i] = 0.0;
    }
    for (int64_t d = 0; d < dim; d++) {
      const int64_t ch = b * dim + d;
      const double* xr = x + ch * L;
      const double* dr = dt + ch * L;
      const double* Bb = B + b * N * L;
      const double* Cb = C + b * N * L;
      const double* Ar = A + d * N;
      const double bias = dt_bias ? dt_bias[d] : 0.0;
      const double Dv = Dskip ? Dskip[d] : 0.0;
      /* forward, keeping every state */
      for (int64_t n = 0; n < N; n++) H[n] = h0 ? h0[ch * N + n] : 0.0;
      for (int64_t t = 0; t < L; t++) {
        const double u = dr[t] + bias;
        const double delta = use_softplus ? sp(u) : u;
        Dl[t] = delta;
        double s = 0.0;
        for (int64_t n = 0; n < N; n++) {
          const double An = Ar[n];
          const double abar = exp(delta * An);
          const double coef = (disc == 0) ? delta : (An == 0.0 ? delta : expm1(delta * An) / An);
          H[(t + 1) * N + n] = abar * H[t * N + n] + coef * Bb[n * L + t] * xr[t];
          s += Cb[n * L + t] * H[(t + 1) * N + n];
        }
        S[t] = s + Dv * xr[t];
      }
      /* backward */
      for (int64_t n = 0; n < N; n++) g[n] = dh_final ? dh_final[ch * N + n] : 0.0;
      double accD = 0.0, accb = 0.0;
      for (int64_t t = L - 1; t >= 0; t--) {
        const double xv = xr[t], dyv = dy[ch * L + t], delta = Dl[t];
        double ds = dyv;
        if (z) {
          const double zv = z[ch * L + t], sg = sigm(zv);
          ds = dyv * zv * sg;
          if (dz) dz[ch * L + t] = dyv * S[t] * (sg * (1.0 + zv * (1.0 - sg)));
        } else if (dz) {
          dz[ch * L + t] = 0.0;
        }
        double dDelta = 0.0, dxv = ds * Dv;
        accD += ds * xv;
        for (int64_t n = 0; n < N; n++) {
          const double An = Ar[n], Bv = Bb[n * L + t], Cv = Cb[n * L + t];
          const double hprev = H[t * N + n], hcur = H[(t + 1) * N + n];
          const double abar = exp(delta * An);
          g[n] += Cv * ds;
          dC[b * N * L + n * L + t] += ds * hcur;
          double coef, dcoef_dd, dcoef_dA;
          if (disc == 0) {
            coef = delta; dcoef_dd = 1.0; dcoef_dA = 0.0;
          } else if (An == 0.0) {
            coef = delta; dcoef_dd = 1.0; dcoef_dA = 0.5 * delta * delta;
          } else {
            const double e = delta * An;
            coef = expm1(e) / An;
            dcoef_dd = abar;
            if (fabs(e) < 1e-3) /* (x e^x - e^x + 1) / x^2 = 1/2 + x/3 + x^2/8 + x^3/30 + ... */
              dcoef_dA = delta * delta * (0.5 + e * (1.0 / 3.0 + e * (1.0 / 8.0 + e * (1.0 / 30.0))));
            else
              dcoef_dA = (delta * abar - coef) / An;
          }
          dDelta += g[n] * (dcoef_dd * Bv * xv + hprev * abar * An);
          dxv += g[n] * coef * Bv;
          dB[b * N * L + n * L + t] += g[n] * coef * xv;
          pA[ch * N + n] += g[n] * (dcoef_dA * Bv * xv + hprev * abar * delta);
          g[n] *= abar;
        }
        const double u = dr[t] + bias;
        const double du = use_softplus ? dDelta * sigm(u) : dDelta;
        ddt[ch * L + t] = du;
        dx[ch * L + t] = dxv;
        accb += du;
      }
      pD[ch] = accD;
      pb[ch] = accb;
      if (dh0)
        for (int64_t n = 0; n < N; n++) dh0[ch * N + n] = g[n];
    }
    free(H); free(Dl); free(S); free(g);
  }
  if (!failed) {
    for (int64_t d = 0; d < dim; d++) {
      double sD = 0.0, sb = 0.0;
      for (int64_t b = 0; b < batch; b++) {
        sD += pD[b * dim + d];
        sb += pb[b * dim + d];
      }
      if (dD) dD[d] = sD;
      if (ddt_bias) ddt_bias[d] = sb;
      for (int64_t n = 0; n < N; n++) {
        double sa = 0.0;
        for (int64_t b = 0; b < batch; b++) sa += pA[(b * dim + d) * N + n];
        dA[d * N + n] = sa;
      }
    }
  }
  free(pA); free(pD); free(pb);
  return failed ? 3 : 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Causal depthwise convolution of width K over the sequence, then SiLU (test infrastructure, fp64).
 * The Mamba block runs it on the SSM branch before the scan (docs.ifdog.com tutorial, "Mamba 架构", step 3a: a
 * depthwise causal 1-D convolution of kernel size d_conv, usually 4, each channel on its own; the SiLU / Swish
 * activation of the block, Mamba paper section 3.4).  Per batch b, channel d, step t:
 *   xc_t = bias[d] + sum_{k=0}^{K-1} w[d][k] * x_{t-(K-1)+k},  x_tau for tau < 0 taken from state_in (oldest first;
 *          zeros when state_in is NULL)
 *   u_t  = silu(xc_t) = xc_t / (1 + exp(-xc_t))   (or xc_t when use_silu == 0)
 *   state_out = the last K-1 inputs x_{L-K+1} .. x_{L-1} (oldest first), continuing from state_in when L < K-1.
 * Layouts: x, u [batch][dim][seqlen]; w [dim][K]; bias [dim]; state_in, state_out [batch][dim][K-1].
 */
int oracle_conv1d_f64(int64_t batch, int64_t dim, int64_t seqlen, int64_t width, int use_silu, const double* x,
                      const double* w, const double* bias, const double* state_in, double* u, double* state_out,
                      int nthreads) {
  if (batch < 0 || dim < 0 || seqlen < 1 || width < 1 || width > 64) return 1;
  if (!x || !w || !u) return 2;
  const int64_t K = width, S = width - 1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel for schedule(static)
  for (int64_t bd = 0; bd < batch * dim; ++bd) {
    const int64_t d = bd % dim;
    const double* xr = x + bd * seqlen;
    const double* st = state_in ? state_in + bd * S : NULL;
    for (int64_t t = 0; t < seqlen; ++t) {
      double acc = bias ? bias[d] : 0.0;
      for (int64_t k = 0; k < K; ++k) {
        const int64_t tau = t - (K - 1) + k;
        const double xv = tau >= 0 ? xr[tau] : (st ? st[S + tau] : 0.0);
        acc += w[d * K + k] * xv;
      }
      u[bd * seqlen + t] = use_silu ? acc / (1.0 + exp(-acc)) : acc;
    }
    if (state_out) {
      double tmp[64];
      for (int64_t i = 0; i < S; ++i) {
        const int64_t tau = seqlen - S + i;
        tmp[i] = tau >= 0 ? xr[tau] : (st ? st[S + tau] : 0.0);
      }
      for (int64_t i = 0; i < S; ++i) state_out[bd * S + i] = tmp[i];
    }
  }
  return 0;
}

/*
 * Backward of oracle_conv1d_f64: the chain rule through u_t = act(pre_t), pre_t = bias + sum_k w[k] e[t + k], where e
 * is the extended input (the K-1 window values of state_in, oldest first, then x).  Given du = dL/du and, optionally,
 * dstate_out = dL/d(state_out) (state_out holds e[L .. L+K-2]):
 *   dpre_t     = du_t act'(pre_t)          act' of SiLU = s (1 + pre (1 - s)) with s = sigmoid(pre); 1 without
 *   de[t + k] += w[k] dpre_t,   de[L + i] += dstate_out[i]
 *   dx[t] = de[K-1 + t],  dstate_in[j] = de[j],  dw[d][k] = sum_b sum_t dpre_t e[t + k],  dbias[d] = sum_b sum_t dpre_t
 * Outputs are overwritten; dbias and dstate_in may be NULL.
 */
int oracle_conv1d_bwd_f64(int64_t batch, int64_t dim, int64_t seqlen, int64_t width, int use_silu, const double* x,
                          const double* w, const double* bias, const double* state_in, const double* du,
                          const double* dstate_out, double* dx, double* dw, double* dbias, double* dstate_in,
                          int nthreads) {
  if (batch < 0 || dim < 0 || seqlen < 1 || width < 1 || width > 64) return 1;
  if (!x || !w || !du || !dx || !dw) return 2;
  const int64_t K = width, S = width - 1, L = seqlen;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  int failed = 0;
#pragma omp parallel for schedule(static)
  for (int64_t d = 0; d < dim; ++d) {
    double* e = (double*)malloc(sizeof(double) * (size_t)(S + L));
    double* de = (double*)malloc(sizeof(double) * (size_t)(S + L));
    if (!e || !de) {
#pragma omp atomic write
      failed = 1;
      free(e); free(de);
      continue;
    }
    double sw[64] = {0.0}, sb = 0.0;
    for (int64_t b = 0; b < batch; ++b) {
      const int64_t bd = b * dim + d;
      for (int64_t j = 0; j < S; ++j) e[j] = state_in ? state_in[bd * S + j] : 0.0;
      for (int64_t t = 0; t < L; ++t) e[S + t] = x[bd * L + t];
      for (int64_t i = 0; i < S + L; ++i) de[i] = 0.0;
      for (int64_t t = 0; t < L; ++t) {
        double pre = bias ? bias[d] : 0.0;
        for (int64_t k = 0; k < K; ++k) pre += w[d * K + k] * e[t + k];
        double g = du[bd * L + t];
        if (use_silu) {
          const double sg = 1.0 / (1.0 + exp(-pre));
          g *= sg * (1.0 + pre * (1.0 - sg));
        }
        for (int64_t k = 0; k < K; ++k) {
          de[t + k] += w[d * K + k] * g;
          sw[k] += g * e[t + k];
        }
        sb += g;
      }
      if (dstate_out)
        for (int64_t i = 0; i < S; ++i) de[L + i] += dstate_out[bd * S + i];
      for (int64_t t = 0; t < L; ++t) dx[bd * L + t] = de[S + t];
      if (dstate_in)
        for (int64_t j = 0; j < S; ++j) dstate_in[bd * S + j] = de[j];
    }
    for (int64_t k = 0; k < K; ++k) dw[d * K + k] = sw[k];
    if (dbias) dbias[d] = sb;
    free(e); free(de);
  }
  return failed ? 3 : 0;
}

/*
 * Complex diagonal A (test infrastructure, fp64).  The Mamba paper (section 3.6, "real vs. complex") keeps a complex
 * state for continuous modalities and initialises A with S4D-Lin, A_n = -1/2 + n i (audio experiments, section 4.4).
 * Same recurrence as oracle_scan_f64 in complex arithmetic, with B and C complex and a real output:
 *   Abar = exp(Delta A)  (complex exponential),  Bbar = Delta B (Euler-B) or (exp(Delta A) - 1) / A * B (ZOH; A = 0
 *   gives Delta B),  h_t = Abar h_{t-1} + Bbar x_t,  y_t = Re(sum_n C_n h_n) + Dskip x_t, times silu(z_t).
 * Complex arrays are interleaved (re, im) on a last axis of 2: A [dim][dstate][2]; B, C [batch][dstate][seqlen][2];
 * h0, h_final, decode state [batch][dim][dstate][2].  x, dt, z, y, dt_bias, Dskip as in oracle_scan_f64.
 */
static void cstep(int64_t N, int disc, int use_softplus, double xv, double dtv, double bias, const double* A_row,
                  const double* Bt, int64_t bstride, const double* Ct, double* h, double* yout) {
  const double u = dtv + bias;
  const double delta = use_softplus ? sp(u) : u;
  double y = 0.0;
  for (int64_t n = 0; n < N; ++n) {
    const double ar = A_row[2 * n], ai = A_row[2 * n + 1];
    const double mag = exp(delta * ar), ang = delta * ai;
    const double abr = mag * cos(ang), abi = mag * sin(ang);  /* Abar = exp(Delta A) */
    const double br = Bt[n * bstride], bi = Bt[n * bstride + 1];
    double cr, ci;                                           /* coefficient of B */
    if (disc == 0 || (ar == 0.0 && ai == 0.0)) {
      cr = delta;
      ci = 0.0;
    } else {                                                 /* (Abar - 1) / A, with expm1 for the real part */
      const double er = expm1(delta * ar) * cos(ang) - 2.0 * sin(0.5 * ang) * sin(0.5 * ang);  /* Re(Abar) - 1 */
      const double ei = abi;
      const double den = ar * ar + ai * ai;
      cr = (er * ar + ei * ai) / den;
      ci = (ei * ar - er * ai) / den;
    }
    const double bbr = (cr * br - ci * bi) * xv, bbi = (cr * bi + ci * br) * xv;
    const double hr = h[2 * n], hi = h[2 * n + 1];
    h[2 * n] = abr * hr - abi * hi + bbr;
    h[2 * n + 1] = abr * hi + abi * hr + bbi;
    y += Ct[n * bstride] * h[2 * n] - Ct[n * bstride + 1] * h[2 * n + 1];
  }
  *yout = y;
}

int oracle_complex_scan_f64(int64_t batch, int64_t dim, int64_t seqlen, int64_t dstate, int disc, int use_softplus,
                            const double* x, const double* dt, const double* dt_bias, const double* A, const double* B,
                            const double* C, const double* Dskip, const double* z, const double* h0, double* y,
                            double* h_final, int nthreads) {
  if (batch < 0 || dim < 0 || seqlen < 1 || dstate < 1 || dstate > 4096) return 1;
  if (!x || !dt || !A || !B || !C || !y) return 2;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  const int64_t N = dstate, L = seqlen;
#pragma omp parallel for schedule(static)
  for (int64_t bd = 0; bd < batch * dim; ++bd) {
    const int64_t b = bd / dim, d = bd % dim;
    double* h = (double*)malloc(sizeof(double) * 2 * (size_t)N);
    for (int64_t i = 0; i < 2 * N; ++i) h[i] = h0 ? h0[bd * 2 * N + i] : 0.0;
    for (int64_t t = 0; t < L; ++t) {
      const double xv = x[bd * L + t];
      double yv;
      cstep(N, disc, use_softplus, xv, dt[bd * L + t], dt_bias ? dt_bias[d] : 0.0, A + d * 2 * N,
            B + (b * N * L + t) * 2, 2 * L, C + (b * N * L + t) * 2, h, &yv);
      if (Dskip) yv += Dskip[d] * xv;
      if (z) {
        const double zv = z[bd * L + t];
        yv *= zv / (1.0 + exp(-zv));
      }
      y[bd * L + t] = yv;
    }
    if (h_final)
      for (int64_t i = 0; i < 2 * N; ++i) h_final[bd * 2 * N + i] = h[i];
    free(h);
  }
  return 0;
}

/* One decode step of oracle_complex_scan_f64; state [batch][dim][dstate][2] updated in place; x, dt, z, y [batch][dim];
 * B, C [batch][dstate][2]. */
int oracle_complex_state_update_f64(int64_t batch, int64_t dim, int64_t dstate, int disc, int use_softplus,
                                    double* state, const double* x, const double* dt, const double* dt_bias,
                                    const double* A, const double* B, const double* C, const double* Dskip,
                                    const double* z, double* y) {
  if (batch < 0 || dim < 0 || dstate < 1) return 1;
  if (!state || !x || !dt || !A || !B || !C || !y) return 2;
  const int64_t N = dstate;
  for (int64_t bd = 0; bd < batch * dim; ++bd) {
    const int64_t b = bd / dim, d = bd % dim;
    double yv;
    cstep(N, disc, use_softplus, x[bd], dt[bd], dt_bias ? dt_bias[d] : 0.0, A + d * 2 * N, B + b * N * 2, 2,
          C + b * N * 2, state + bd * 2 * N, &yv);
    if (Dskip) yv += Dskip[d] * x[bd];
    if (z) yv *= z[bd] / (1.0 + exp(-z[bd]));
    y[bd] = yv;
  }
  return 0;
}


/*
 * Mamba-2 / state space duality (SSD) layer: the same selective recurrence with the state matrix reduced to a scalar
 * times the identity per head, and a head structure like multi-head attention (close reading, section on Mamba-2
 * and SSD; tutorial, "Mamba-2 与结构化对偶性": larger states such as N = 128 or 256).  nheads heads of width headdim
 * split the channels; head h reads B and C of group g = h / (nheads / ngroups).  Per batch b, head h, column p the
 * state is a row S[0..N-1]:
 *   u     = dt[b,t,h] + dt_bias[h];  Delta = softplus(u) (or u)
 *   abar  = exp(Delta * A[h])                       (one scalar per head and step)
 *   coef  = Delta (Euler rule)  or  expm1(Delta*A[h]) / A[h]  (zero-order hold; Delta when A[h] == 0)
 *   S[n]  = abar * S[n] + coef * B[b,t,g,n] * x[b,t,h,p]
 *   y[b,t,h,p] = sum_n C[b,t,g,n] * S[n] + D[h] * x[b,t,h,p],  times silu(z[b,t,h,p]) when z is given
 * This is the recurrent form.  Its dual, the masked quadratic form y = (L o C B^T)(coef x) with the decay mask
 * L[t,s] = exp(A * (cum_t - cum_s)) for s <= t, is what the pins compare it against; it is not used here.
 * Layouts (fp64, row-major): x, z, y: [batch][seqlen][nheads][headdim]; dt: [batch][seqlen][nheads];
 * B, C: [batch][seqlen][ngroups][dstate]; A, dt_bias, D: [nheads]; h0, h_final and the decode state:
 * [batch][nheads][headdim][dstate].
 */
int oracle_ssd_f64(int64_t batch, int64_t seqlen, int64_t nheads, int64_t headdim, int64_t ngroups, int64_t dstate,
                   int disc, int use_softplus, const double* x, const double* dt, const double* dt_bias,
                   const double* A, const double* B, const double* C, const double* Dskip, const double* z,
                   const double* h0, double* y, double* h_final, int nthreads) {
  if (batch < 1 || seqlen < 0 || nheads < 1 || headdim < 1 || ngroups < 1 || dstate < 1 || dstate > 4096 ||
      nheads % ngroups)
    return 1;
  if (!x || !dt || !A || !B || !C || !y) return 2;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  const int64_t H = nheads, P = headdim, N = dstate, G = ngroups, hpg = nheads / ngroups;
  const int64_t nch = batch * H * P;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t ch = 0; ch < nch; ch++) {
    const int64_t b = ch / (H * P), h = (ch / P) % H, p = ch % P, g = h / hpg;
    double S[4096];
    for (int64_t n = 0; n < N; n++) S[n] = h0 ? h0[ch * N + n] : 0.0;
    const double Ah = A[h];
    for (int64_t t = 0; t < seqlen; t++) {
      const int64_t row = (b * seqlen + t) * H + h;          /* index of (b, t, h) */
      const double xv = x[row * P + p];
      const double u = dt[row] + (dt_bias ? dt_bias[h] : 0.0);
      const double delta = use_softplus ? sp(u) : u;
      const double abar = exp(delta * Ah);
      const double coef = disc == 0 ? delta : (Ah == 0.0 ? delta : expm1(delta * Ah) / Ah);
      const double* Bt = B + ((b * seqlen + t) * G + g) * N;
      const double* Ct = C + ((b * seqlen + t) * G + g) * N;
      double acc = 0.0;
      for (int64_t n = 0; n < N; n++) {
        S[n] = abar * S[n] + coef * Bt[n] * xv;
        acc += Ct[n] * S[n];
      }
      if (Dskip) acc += Dskip[h] * xv;
      if (z) {
        const double zv = z[row * P + p];
        acc *= zv / (1.0 + exp(-zv));
      }
      y[row * P + p] = acc;
    }
    if (h_final)
      for (int64_t n = 0; n < N; n++) h_final[ch * N + n] = S[n];
  }
  return 0;
}

/* One SSD decode step: state [batch][nheads][headdim][dstate] updated in place; x, z, y: [batch][nheads][headdim];
 * dt: [batch][nheads]; B, C: [batch][ngroups][dstate].  The same body as oracle_ssd_f64 for a single t. */
int oracle_ssd_state_update_f64(int64_t batch, int64_t nheads, int64_t headdim, int64_t ngroups, int64_t dstate,
                                int disc, int use_softplus, double* state, const double* x, const double* dt,
                                const double* dt_bias, const double* A, const double* B, const double* C,
                                const double* Dskip, const double* z, double* y) {
  if (batch < 1 || nheads < 1 || headdim < 1 || ngroups < 1 || dstate < 1 || nheads % ngroups) return 1;
  if (!state || !x || !dt || !A || !B || !C || !y) return 2;
  const int64_t H = nheads, P = headdim, N = dstate, G = ngroups, hpg = nheads / ngroups;
  for (int64_t b = 0; b < batch; b++)
    for (int64_t h = 0; h < H; h++) {
      const int64_t g = h / hpg;
      const double Ah = A[h];
      const double u = dt[b * H + h] + (dt_bias ? dt_bias[h] : 0.0);
      const double delta = use_softplus ? sp(u) : u;
      const double abar = exp(delta * Ah);
      const double coef = disc == 0 ? delta : (Ah == 0.0 ? delta : expm1(delta * Ah) / Ah);
      const double* Bt = B + (b * G + g) * N;
      const double* Ct = C + (b * G + g) * N;
      for (int64_t p = 0; p < P; p++) {
        const int64_t i = (b * H + h) * P + p;
        double* S = state + i * N;
        double acc = 0.0;
        for (int64_t n = 0; n < N; n++) {
          S[n] = abar * S[n] + coef * Bt[n] * x[i];
          acc += Ct[n] * S[n];
        }
        if (Dskip) acc += Dskip[h] * x[i];
        if (z) acc *= z[i] / (1.0 + exp(-z[i]));
        y[i] = acc;
      }
    }
  return 0;
}
