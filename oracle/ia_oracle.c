/*
 * ia_oracle.c — TEST INFRASTRUCTURE, not part of the product.
 *
 * A plain, serial, fp64 CPU implementation of one Interdomain Attention (IA) layer, written
 * to be checked against the pages by eye.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg load it.  It shares no code with the HIP library.
 *
 * What it follows (the two pages titled "Interdomain Attention: Beyond Token-Level Key-Value
 * Memory": the paper summary page and the AI Radio episode page):
 *   - feature map phi(x) = elu(x)+1 and the finite-feature kernel K(q,k) ~ phi(q)^T phi(k)
 *     (episode page, "Key Components and Derivation");
 *   - key features and values projected onto M modes by a complex-diagonal S4D recurrence
 *     (summary §3.1, §3.2; episode page, derivation): for every mode m
 *         U[m,:]   <- lambda_m U[m,:]   + beta_m phi(k_t)
 *         Gam[m,:] <- lambda_m Gam[m,:] + beta_m v_t
 *         eta[m]   <- lambda_m eta[m]   + beta_m
 *   - the readout of the matrix form O = Fq U^T Gamma / Fq U^T eta, division element-wise
 *     (episode page, derivation): a[m] = sum_r phi(q_t)[r] U[m,r] (transpose, no conjugate),
 *     num = Re sum_m a[m] Gam[m,:], den = Re sum_m a[m] eta[m], o_t = num / max(den, clamp).
 *   Readings where the pages are silent: the readout at step t uses the state after token t
 *   is added; Re() is taken of the numerator and of the denominator separately; the clamp is
 *   one-sided (den below clamp, negative included, becomes clamp).
 *
 * The state is complex128 here; inputs arrive as float64 arrays holding exactly the values
 * the GPU receives (bf16- or fp32-rounded q, k, v; complex64-rounded lambda and beta).
 *
 * Built with: gcc -O2 -ffp-contract=off -fPIC -shared (no fast-math), so that every product
 * and sum is rounded as written.
 */
#include <complex.h>
#include <math.h>
#include <stddef.h>
#include <stdlib.h>

static double feature(double x) {
  /* elu(x) + 1: x + 1 for x > 0, exp(x) for x <= 0 */
  return x > 0.0 ? x + 1.0 : exp(x);
}

/*
 * One (b,h) slice, tokens t = 0..N-1 in order.
 *   q, k     [N][F]    raw inputs (the feature map is applied here)
 *   v        [N][D]
 *   lam,beta [M][2]    (re, im)
 *   U        [M][F][2] state in/out
 *   G        [M][D][2] state in/out
 *   e        [M][2]    state in/out
 *   o        [N][D]    outputs, or NULL
 *   num      [N][D]    Re numerator, or NULL
 *   den      [N]       Re denominator before the clamp, or NULL
 * Returns 0.
 */
int ia_oracle_scan(int N, int F, int D, int M,
                   const double* q, const double* k, const double* v,
                   const double* lam, const double* beta,
                   double* U, double* G, double* e,
                   double* o, double* num, double* den, double clamp) {
  for (int t = 0; t < N; ++t) {
    const double* qt = q + (size_t)t * F;
    const double* kt = k + (size_t)t * F;
    const double* vt = v + (size_t)t * D;
    double complex numc[D];
    for (int j = 0; j < D; ++j) numc[j] = 0.0;
    double complex denc = 0.0;

    for (int m = 0; m < M; ++m) {
      double complex l = lam[2 * m] + I * lam[2 * m + 1];
      double complex bm = beta[2 * m] + I * beta[2 * m + 1];

      /* U[m,:] <- lambda_m U[m,:] + beta_m phi(k_t), then a[m] = phi(q_t) . U[m,:] */
      double complex a = 0.0;
      for (int r = 0; r < F; ++r) {
        double* u = U + ((size_t)m * F + r) * 2;
        double complex uc = u[0] + I * u[1];
        uc = l * uc + bm * feature(kt[r]);
        u[0] = creal(uc);
        u[1] = cimag(uc);
        a += feature(qt[r]) * uc;
      }

      /* Gam[m,:] <- lambda_m Gam[m,:] + beta_m v_t, accumulate a[m] Gam[m,:] */
      for (int j = 0; j < D; ++j) {
        double* g = G + ((size_t)m * D + j) * 2;
        double complex gc = g[0] + I * g[1];
        gc = l * gc + bm * vt[j];
        g[0] = creal(gc);
        g[1] = cimag(gc);
        numc[j] += a * gc;
      }

      /* eta[m] <- lambda_m eta[m] + beta_m, accumulate a[m] eta[m] */
      double complex ec = e[2 * m] + I * e[2 * m + 1];
      ec = l * ec + bm;
      e[2 * m] = creal(ec);
      e[2 * m + 1] = cimag(ec);
      denc += a * ec;
    }

    double d = creal(denc);
    double dc = d < clamp ? clamp : d;
    if (isnan(d)) dc = d; /* NaN propagates */
    if (den) den[t] = d;
    for (int j = 0; j < D; ++j) {
      double n = creal(numc[j]);
      if (num) num[(size_t)t * D + j] = n;
      if (o) o[(size_t)t * D + j] = n / dc;
    }
  }
  return 0;
}

/*
 * Gradients of one (b,h) slice of the layer above, by reverse-mode differentiation of the same
 * recurrence: given dL/do for every output, the gradients of a real loss L with respect to q,
 * k, v, lambda, beta and the initial state.  The training-time claims of the summary page
 * (§G: a training step is the forward and this backward) are what it serves.
 *
 * Convention for a complex quantity z (lambda, beta, the state): its gradient is
 * dL/dRe z + i dL/dIm z.  With that convention, for w = p z (p fixed) the gradient of z
 * gathers conj(p) times that of w, and for real x with w = x u it gathers Re(g_w conj(u)).
 *
 * Plainly: a forward sweep keeps every state U_t, Gam_t, eta_t (t = -1 for the initial
 * state), a_t, num_t and den_t; a reverse sweep then carries the state adjoints
 *   Ubar_t = (readout at t) + conj(lambda) Ubar_{t+1}   (the same for Gam and eta)
 * and collects every input's gradient at the step that uses it.  The readout
 * o = num / max(den, clamp) differentiates to dnum = g / c and, when den >= clamp (the
 * branch the forward takes for den itself), dden = -sum_j g_j num_j / c^2; below the clamp
 * dden = 0.  With no_den != 0 the output is num itself: dnum = g, dden = 0.
 *
 *   dO        [N][D]       dL/do
 *   U0,G0,e0  initial state as in ia_oracle_scan, or NULL for zeros
 *   dq, dk    [N][F]       out: dL/dq, dL/dk (through phi' = 1 above 0, exp(x) at or below)
 *   dv        [N][D]       out
 *   dlam,dbeta [M][2]      out: complex gradients as above
 *   dU0,dG0,de0            out: gradients of the initial state, or NULL
 *   work      (N+1) * M * (F+D+1) * 2 + N * M * 2 + N * (D+1) doubles
 * Returns 0.
 */
static double feature_grad(double x) { return x > 0.0 ? 1.0 : exp(x); }

int ia_oracle_scan_bwd(int N, int F, int D, int M,
                       const double* q, const double* k, const double* v,
                       const double* lam, const double* beta,
                       const double* U0, const double* G0, const double* e0,
                       const double* dO, double clamp, int no_den,
                       double* dq, double* dk, double* dv, double* dlam, double* dbeta,
                       double* dU0, double* dG0, double* de0, double* work) {
  const size_t SU = (size_t)M * F, SG = (size_t)M * D;   /* complex entries per state */
  double complex* Us = (double complex*)work;              /* [N+1][M][F], slot t+1 = U_t */
  double complex* Gs = Us + (size_t)(N + 1) * SU;          /* [N+1][M][D] */
  double complex* es = Gs + (size_t)(N + 1) * SG;          /* [N+1][M] */
  double complex* as = es + (size_t)(N + 1) * M;           /* [N][M] */
  double* nums = (double*)(as + (size_t)N * M);            /* [N][D] */
  double* dens = nums + (size_t)N * D;                     /* [N] */

  /* forward sweep, every state kept */
  for (size_t i = 0; i < SU; ++i) Us[i] = U0 ? U0[2 * i] + I * U0[2 * i + 1] : 0.0;
  for (size_t i = 0; i < SG; ++i) Gs[i] = G0 ? G0[2 * i] + I * G0[2 * i + 1] : 0.0;
  for (int m = 0; m < M; ++m) es[m] = e0 ? e0[2 * m] + I * e0[2 * m + 1] : 0.0;
  for (int t = 0; t < N; ++t) {
    const double complex* Up = Us + (size_t)t * SU;
    const double complex* Gp = Gs + (size_t)t * SG;
    const double complex* ep = es + (size_t)t * M;
    double complex* Un = Us + (size_t)(t + 1) * SU;
    double complex* Gn = Gs + (size_t)(t + 1) * SG;
    double complex* en = es + (size_t)(t + 1) * M;
    double complex denc = 0.0;
    for (int j = 0; j < D; ++j) nums[(size_t)t * D + j] = 0.0;
    for (int m = 0; m < M; ++m) {
      const double complex lm = lam[2 * m] + I * lam[2 * m + 1];
      const double complex bt = beta[2 * m] + I * beta[2 * m + 1];
      double complex a = 0.0;
      for (int r = 0; r < F; ++r) {
        const size_t i = (size_t)m * F + r;
        Un[i] = lm * Up[i] + bt * feature(k[(size_t)t * F + r]);
        a += feature(q[(size_t)t * F + r]) * Un[i];
      }
      as[(size_t)t * M + m] = a;
      for (int j = 0; j < D; ++j) {
        const size_t i = (size_t)m * D + j;
        Gn[i] = lm * Gp[i] + bt * v[(size_t)t * D + j];
        nums[(size_t)t * D + j] += creal(a * Gn[i]);
      }
      en[m] = lm * ep[m] + bt;
      denc += a * en[m];
    }
    dens[t] = creal(denc);
  }

  /* reverse sweep: Ub, Gb, eb hold the adjoints of U_t, Gam_t, eta_t */
  double complex* Ub = (double complex*)calloc(SU + SG + M, sizeof(double complex));
  if (!Ub) return 1;
  double complex* Gb = Ub + SU;
  double complex* eb = Gb + SG;
  for (int m = 0; m < M; ++m) { dlam[2 * m] = dlam[2 * m + 1] = 0.0; dbeta[2 * m] = dbeta[2 * m + 1] = 0.0; }
  for (int t = N - 1; t >= 0; --t) {
    const double* g = dO + (size_t)t * D;
    const double d = dens[t];
    double c = d < clamp ? clamp : d;
    if (isnan(d)) c = d;
    double dnum_scale, dden;
    if (no_den) {
      dnum_scale = 1.0;
      dden = 0.0;
    } else {
      double gn = 0.0;
      for (int j = 0; j < D; ++j) gn += g[j] * nums[(size_t)t * D + j];
      dnum_scale = 1.0 / c;
      dden = d >= clamp ? -gn / (c * c) : 0.0;
    }
    const double complex* Ut = Us + (size_t)(t + 1) * SU;
    const double complex* Gt = Gs + (size_t)(t + 1) * SG;
    const double complex* et = es + (size_t)(t + 1) * M;
    const double complex* Up = Us + (size_t)t * SU;
    const double complex* Gp = Gs + (size_t)t * SG;
    const double complex* ep = es + (size_t)t * M;
    for (int r = 0; r < F; ++r) dq[(size_t)t * F + r] = dk[(size_t)t * F + r] = 0.0;
    for (int j = 0; j < D; ++j) dv[(size_t)t * D + j] = 0.0;
    for (int m = 0; m < M; ++m) {
      const double complex lm = lam[2 * m] + I * lam[2 * m + 1];
      const double complex bt = beta[2 * m] + I * beta[2 * m + 1];
      const double complex a = as[(size_t)t * M + m];
      /* readout: num_j = Re sum_m a_m Gam_mj, den = Re sum_m a_m eta_m */
      double complex ga = dden * conj(et[m]);                  /* gradient of a_m */
      for (int j = 0; j < D; ++j) {
        const size_t i = (size_t)m * D + j;
        const double dn = dnum_scale * g[j];
        ga += dn * conj(Gt[i]);
        Gb[i] += dn * conj(a);
      }
      eb[m] += dden * conj(a);
      /* a_m = sum_r phi(q_r) U_mr */
      for (int r = 0; r < F; ++r) {
        const size_t i = (size_t)m * F + r;
        dq[(size_t)t * F + r] += creal(ga * conj(Ut[i]));
        Ub[i] += feature(q[(size_t)t * F + r]) * ga;
      }
      /* U_t = lambda U_{t-1} + beta phi(k_t), and the same for Gam (with v_t) and eta (with 1) */
      double complex gl = 0.0, gb = 0.0;
      for (int r = 0; r < F; ++r) {
        const size_t i = (size_t)m * F + r;
        const double fk = feature(k[(size_t)t * F + r]);
        dk[(size_t)t * F + r] += creal(Ub[i] * conj(bt));
        gb += Ub[i] * fk;
        gl += Ub[i] * conj(Up[i]);
        Ub[i] = conj(lm) * Ub[i];
      }
      for (int j = 0; j < D; ++j) {
        const size_t i = (size_t)m * D + j;
        dv[(size_t)t * D + j] += creal(Gb[i] * conj(bt));
        gb += Gb[i] * v[(size_t)t * D + j];
        gl += Gb[i] * conj(Gp[i]);
        Gb[i] = conj(lm) * Gb[i];
      }
      gb += eb[m];
      gl += eb[m] * conj(ep[m]);
      eb[m] = conj(lm) * eb[m];
      dlam[2 * m] += creal(gl);
      dlam[2 * m + 1] += cimag(gl);
      dbeta[2 * m] += creal(gb);
      dbeta[2 * m + 1] += cimag(gb);
    }
    for (int r = 0; r < F; ++r) {
      dq[(size_t)t * F + r] *= feature_grad(q[(size_t)t * F + r]);
      dk[(size_t)t * F + r] *= feature_grad(k[(size_t)t * F + r]);
    }
  }
  /* what is left in the adjoints is the gradient of the initial state */
  for (size_t i = 0; i < SU; ++i) if (dU0) { dU0[2 * i] = creal(Ub[i]); dU0[2 * i + 1] = cimag(Ub[i]); }
  for (size_t i = 0; i < SG; ++i) if (dG0) { dG0[2 * i] = creal(Gb[i]); dG0[2 * i + 1] = cimag(Gb[i]); }
  for (int m = 0; m < M; ++m) if (de0) { de0[2 * m] = creal(eb[m]); de0[2 * m + 1] = cimag(eb[m]); }
  free(Ub);
  return 0;
}

/*
 * The same layer with a learned complex M x M readout matrix R between phi(q_t) U^T and Gamma
 * (the full readout matrix listed with the practical layer's dimensions, summary page §A.3,
 * whose cost per decode step is the M^2 term of §3.2).  Reading: R mixes the modes of a before
 * both readouts, a'[n] = sum_m a[m] R[m][n], num = Re sum_n a'[n] Gam[n,:],
 * den = Re sum_n a'[n] eta[n], o = num / max(den, clamp); R = identity is the layer above.
 *   R   [M][M][2] (re, im), row m, column n.  Other arguments as ia_oracle_scan.
 *   work  M * 4 doubles.
 * Returns 0.
 */
int ia_oracle_scan_readout(int N, int F, int D, int M,
                           const double* q, const double* k, const double* v,
                           const double* lam, const double* beta, const double* R,
                           double* U, double* G, double* e,
                           double* o, double* num, double* den, double clamp, double* work) {
  double complex* av = (double complex*)work;   /* a[m] */
  double complex* ar = av + M;                  /* (a R)[n] */
  for (int t = 0; t < N; ++t) {
    /* every state row advanced by token t; a[m] = phi(q_t) . U[m,:] */
    for (int m = 0; m < M; ++m) {
      const double complex lm = lam[2 * m] + I * lam[2 * m + 1];
      const double complex bt = beta[2 * m] + I * beta[2 * m + 1];
      double complex acc = 0.0;
      for (int r = 0; r < F; ++r) {
        double* u = U + ((size_t)m * F + r) * 2;
        const double complex uc = lm * (u[0] + I * u[1]) + bt * feature(k[(size_t)t * F + r]);
        u[0] = creal(uc);
        u[1] = cimag(uc);
        acc += feature(q[(size_t)t * F + r]) * uc;
      }
      av[m] = acc;
      for (int j = 0; j < D; ++j) {
        double* g = G + ((size_t)m * D + j) * 2;
        const double complex gc = lm * (g[0] + I * g[1]) + bt * v[(size_t)t * D + j];
        g[0] = creal(gc);
        g[1] = cimag(gc);
      }
      const double complex ec = lm * (e[2 * m] + I * e[2 * m + 1]) + bt;
      e[2 * m] = creal(ec);
      e[2 * m + 1] = cimag(ec);
    }
    for (int n = 0; n < M; ++n) {
      double complex acc = 0.0;
      for (int m = 0; m < M; ++m)
        acc += av[m] * (R[((size_t)m * M + n) * 2] + I * R[((size_t)m * M + n) * 2 + 1]);
      ar[n] = acc;
    }
    double complex dc = 0.0;
    for (int n = 0; n < M; ++n) dc += ar[n] * (e[2 * n] + I * e[2 * n + 1]);
    const double d = creal(dc);
    double c = d < clamp ? clamp : d;
    if (isnan(d)) c = d;
    if (den) den[t] = d;
    for (int j = 0; j < D; ++j) {
      double complex nc = 0.0;
      for (int n = 0; n < M; ++n) {
        const double* g = G + ((size_t)n * D + j) * 2;
        nc += ar[n] * (g[0] + I * g[1]);
      }
      if (num) num[(size_t)t * D + j] = creal(nc);
      if (o) o[(size_t)t * D + j] = creal(nc) / c;
    }
  }
  return 0;
}

/*
 * The layer with selective writing and memory decay: the optional enhancement in which
 * input-dependent gates control what the memory stores and how fast it forgets (summary page
 * §3.3; ablated as selective vs non-selective in §B.3, Table 7).  The pages give no formula;
 * the reading taken here, per token t of the slice, with two real gates the caller computes
 * from the input:
 *   write gate  w_t  scales what token t writes into every memory (U, Gam and eta alike);
 *   decay gate  a_t  scales every mode's lambda at step t (0 < a_t <= 1 forgets faster).
 * For every mode m
 *     U[m,:]   <- a_t lambda_m U[m,:]   + w_t beta_m phi(k_t)
 *     Gam[m,:] <- a_t lambda_m Gam[m,:] + w_t beta_m v_t
 *     eta[m]   <- a_t lambda_m eta[m]   + w_t beta_m
 * and the readout of ia_oracle_scan, unchanged.  w = a = 1 is the plain layer.
 *   wgate, dgate  [N]  write and decay gates of the slice's tokens
 * Other arguments as ia_oracle_scan.  Returns 0.
 */
int ia_oracle_scan_gated(int N, int F, int D, int M,
                         const double* q, const double* k, const double* v,
                         const double* lam, const double* beta,
                         const double* wgate, const double* dgate,
                         double* U, double* G, double* e,
                         double* o, double* num, double* den, double clamp) {
  for (int t = 0; t < N; ++t) {
    const double w = wgate[t], at = dgate[t];
    double complex nsum[D];
    for (int j = 0; j < D; ++j) nsum[j] = 0.0;
    double complex dsum = 0.0;
    for (int m = 0; m < M; ++m) {
      const double complex l = at * (lam[2 * m] + I * lam[2 * m + 1]);
      const double complex wb = w * (beta[2 * m] + I * beta[2 * m + 1]);
      double complex a = 0.0;
      for (int r = 0; r < F; ++r) {
        double* u = U + ((size_t)m * F + r) * 2;
        const double complex uc = l * (u[0] + I * u[1]) + wb * feature(k[(size_t)t * F + r]);
        u[0] = creal(uc);
        u[1] = cimag(uc);
        a += feature(q[(size_t)t * F + r]) * uc;
      }
      for (int j = 0; j < D; ++j) {
        double* g = G + ((size_t)m * D + j) * 2;
        const double complex gc = l * (g[0] + I * g[1]) + wb * v[(size_t)t * D + j];
        g[0] = creal(gc);
        g[1] = cimag(gc);
        nsum[j] += a * gc;
      }
      const double complex ec = l * (e[2 * m] + I * e[2 * m + 1]) + wb;
      e[2 * m] = creal(ec);
      e[2 * m + 1] = cimag(ec);
      dsum += a * ec;
    }
    const double dr = creal(dsum);
    double c = dr < clamp ? clamp : dr;
    if (isnan(dr)) c = dr;
    if (den) den[t] = dr;
    for (int j = 0; j < D; ++j) {
      const double n = creal(nsum[j]);
      if (num) num[(size_t)t * D + j] = n;
      if (o) o[(size_t)t * D + j] = n / c;
    }
  }
  return 0;
}
