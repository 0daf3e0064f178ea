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
