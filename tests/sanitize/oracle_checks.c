/* The oracle's functions on small random inputs under AddressSanitizer and
 * UndefinedBehaviorSanitizer: every buffer sized as its header comment states.  Exit status
 * 0 when the runs finish and unit gates reproduce the plain scan exactly. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int ia_oracle_scan(int, int, int, int, const double*, const double*, const double*,
                   const double*, const double*, double*, double*, double*, double*, double*,
                   double*, double);
int ia_oracle_scan_gated(int, int, int, int, const double*, const double*, const double*,
                         const double*, const double*, const double*, const double*, double*,
                         double*, double*, double*, double*, double*, double);
int ia_oracle_scan_readout(int, int, int, int, const double*, const double*, const double*,
                           const double*, const double*, const double*, double*, double*,
                           double*, double*, double*, double*, double, double*);
int ia_oracle_scan_bwd(int, int, int, int, const double*, const double*, const double*,
                       const double*, const double*, const double*, const double*,
                       const double*, const double*, double, int, double*, double*, double*,
                       double*, double*, double*, double*, double*, double*);

static double* rnd(size_t n, unsigned* seed) {
  double* p = malloc(n * sizeof(double));
  for (size_t i = 0; i < n; ++i) p[i] = (double)rand_r(seed) / RAND_MAX - 0.5;
  return p;
}

int main(void) {
  unsigned seed = 7;
  const int N = 13, F = 5, D = 6, M = 4;
  double *q = rnd((size_t)N * F, &seed), *k = rnd((size_t)N * F, &seed);
  double *v = rnd((size_t)N * D, &seed), *lam = rnd(2 * M, &seed), *beta = rnd(2 * M, &seed);
  double *R = rnd(2 * (size_t)M * M, &seed), *dO = rnd((size_t)N * D, &seed);
  double *U0 = rnd(2 * (size_t)M * F, &seed), *G0 = rnd(2 * (size_t)M * D, &seed);
  double *e0 = rnd(2 * M, &seed);
  double *ones = malloc(N * sizeof(double));
  for (int t = 0; t < N; ++t) ones[t] = 1.0;
  double *U = malloc(2 * (size_t)M * F * sizeof(double)), *G = malloc(2 * (size_t)M * D * sizeof(double));
  double *e = malloc(2 * M * sizeof(double));
  double *o1 = malloc((size_t)N * D * sizeof(double)), *o2 = malloc((size_t)N * D * sizeof(double));
  double *num = malloc((size_t)N * D * sizeof(double)), *den = malloc(N * sizeof(double));
  memcpy(U, U0, 2 * (size_t)M * F * sizeof(double));
  memcpy(G, G0, 2 * (size_t)M * D * sizeof(double));
  memcpy(e, e0, 2 * M * sizeof(double));
  ia_oracle_scan(N, F, D, M, q, k, v, lam, beta, U, G, e, o1, num, den, 1e-6);
  memcpy(U, U0, 2 * (size_t)M * F * sizeof(double));
  memcpy(G, G0, 2 * (size_t)M * D * sizeof(double));
  memcpy(e, e0, 2 * M * sizeof(double));
  ia_oracle_scan_gated(N, F, D, M, q, k, v, lam, beta, ones, ones, U, G, e, o2, num, den, 1e-6);
  int bad = memcmp(o1, o2, (size_t)N * D * sizeof(double)) != 0;
  double* work = malloc(4 * M * sizeof(double));
  ia_oracle_scan_readout(N, F, D, M, q, k, v, lam, beta, R, U, G, e, o1, num, den, 1e-6, work);
  const size_t nw = (size_t)(N + 1) * M * (F + D + 1) * 2 + (size_t)N * M * 2 + (size_t)N * (D + 1);
  double* bw = malloc(nw * sizeof(double));
  double *dq = malloc((size_t)N * F * sizeof(double)), *dk = malloc((size_t)N * F * sizeof(double));
  double *dv = malloc((size_t)N * D * sizeof(double)), *dl = malloc(2 * M * sizeof(double));
  double *db = malloc(2 * M * sizeof(double)), *dU = malloc(2 * (size_t)M * F * sizeof(double));
  double *dG = malloc(2 * (size_t)M * D * sizeof(double)), *de = malloc(2 * M * sizeof(double));
  ia_oracle_scan_bwd(N, F, D, M, q, k, v, lam, beta, U0, G0, e0, dO, 1e-6, 0, dq, dk, dv, dl, db,
                     dU, dG, de, bw);
  ia_oracle_scan_bwd(N, F, D, M, q, k, v, lam, beta, NULL, NULL, NULL, dO, 1e-6, 1, dq, dk, dv,
                     dl, db, NULL, NULL, NULL, bw);
  free(q); free(k); free(v); free(lam); free(beta); free(R); free(dO); free(U0); free(G0);
  free(e0); free(ones); free(U); free(G); free(e); free(o1); free(o2); free(num); free(den);
  free(work); free(bw); free(dq); free(dk); free(dv); free(dl); free(db); free(dU); free(dG);
  free(de);
  printf("%s\n", bad ? "FAILED: unit gates differ from the plain scan" : "ok");
  return bad;
}
