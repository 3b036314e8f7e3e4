/*
 * Host sanitizer driver for the fp64 oracle (built with gcc and
 * -fsanitize=address,undefined together with oracle/efla_oracle.c; CPU only,
 * test infrastructure). It runs every exported oracle routine on small
 * inputs, including a ragged multi-threaded call, and checks a few
 * properties that hold exactly: a zero step size leaves the state unchanged,
 * and the forward's per-step norm at the last token equals the norm of the
 * final state. Exit status 0 means no sanitizer report and no failed check.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double efla_oracle_alpha(double beta, double lam);
double efla_oracle_coef(int mode, double beta, double lam);
void efla_oracle_step(int mode, const double* q, const double* k, const double* v, double beta,
                      double* S, double* o, int dk, int dv);
int efla_oracle_fwd(int mode, const double* q, const double* k, const double* v,
                    const double* beta, const double* s0, double* o, double* s_final,
                    double* snorm, long nh, long T, int dk, int dv, int nthreads);
void efla_oracle_coef_grad(int mode, double beta, double lam, double* dbeta, double* dlam);
void efla_oracle_step_gated(int mode, const double* q, const double* k, const double* v, double beta,
                            double log_g, double* S, double* o, int dk, int dv);
int efla_oracle_fwd_gated(int mode, const double* q, const double* k, const double* v,
                          const double* beta, const double* log_g, const double* s0, double* o,
                          double* s_final, long nh, long T, int dk, int dv, int nthreads);
int efla_oracle_bwd(int mode, const double* q, const double* k, const double* v,
                    const double* beta, const double* s0, const double* dout, const double* dsT,
                    double* dq, double* dk, double* dv, double* dbeta, double* ds0, long nh,
                    long T, int dk_, int dv_, int nthreads);

static double urand(unsigned* s) {
  *s = *s * 1664525u + 1013904223u;
  return (double)(*s >> 8) / 16777216.0 - 0.5;
}

static double* fill(size_t n, unsigned* s, double scale) {
  double* p = (double*)malloc(n * sizeof(double));
  for (size_t i = 0; i < n; ++i) p[i] = scale * urand(s);
  return p;
}

int main(void) {
  unsigned seed = 12345u;
  const long nh = 5, T = 37;
  const int dk = 6, dv = 4;
  int fails = 0;
  double* q = fill((size_t)nh * T * dk, &seed, 2.0);
  double* k = fill((size_t)nh * T * dk, &seed, 4.0);
  double* v = fill((size_t)nh * T * dv, &seed, 2.0);
  double* beta = fill((size_t)nh * T, &seed, 1.0);
  double* s0 = fill((size_t)nh * dk * dv, &seed, 1.0);
  double* dout = fill((size_t)nh * T * dv, &seed, 1.0);
  double* dsT = fill((size_t)nh * dk * dv, &seed, 1.0);
  for (long i = 0; i < nh * T; ++i) beta[i] += 0.5;
  double* o = (double*)calloc((size_t)nh * T * dv, sizeof(double));
  double* sf = (double*)calloc((size_t)nh * dk * dv, sizeof(double));
  double* sn = (double*)calloc((size_t)nh * T, sizeof(double));

  for (int mode = 0; mode < 4; ++mode) {
    (void)efla_oracle_alpha(0.7, 1e-14);
    (void)efla_oracle_coef(mode, 0.3, 2.0);
    double gb, gl;
    efla_oracle_coef_grad(mode, 0.3, 2.0, &gb, &gl);
    for (int th = 1; th <= 3; ++th) {
      if (efla_oracle_fwd(mode, q, k, v, beta, th == 2 ? NULL : s0, o, sf, sn, nh, T, dk, dv, th) != 0)
        ++fails;
      for (long h = 0; h < nh; ++h) {
        double n2 = 0.0;
        for (int e = 0; e < dk * dv; ++e) n2 += sf[h * dk * dv + e] * sf[h * dk * dv + e];
        if (fabs(sqrt(n2) - sn[h * T + T - 1]) > 1e-12 * (1.0 + sqrt(n2))) ++fails;
      }
    }
    double *gq = calloc((size_t)nh * T * dk, 8), *gk = calloc((size_t)nh * T * dk, 8),
           *gv = calloc((size_t)nh * T * dv, 8), *gbt = calloc((size_t)nh * T, 8),
           *gs = calloc((size_t)nh * dk * dv, 8);
    if (efla_oracle_bwd(mode, q, k, v, beta, s0, dout, dsT, gq, gk, gv, gbt, gs, nh, T, dk, dv, 2) != 0) ++fails;
    if (efla_oracle_bwd(mode, q, k, v, beta, NULL, dout, NULL, gq, gk, gv, gbt, gs, nh, T, dk, dv, 3) != 0) ++fails;
    free(gq), free(gk), free(gv), free(gbt), free(gs);
  }
  /* beta = 0: the state never changes */
  double* z = (double*)calloc((size_t)nh * T, sizeof(double));
  efla_oracle_fwd(0, q, k, v, z, s0, o, sf, NULL, nh, T, dk, dv, 2);
  if (memcmp(sf, s0, sizeof(double) * (size_t)nh * dk * dv) != 0) ++fails;
  /* gated variant: zero log-decays reproduce the ungated forward to rounding */
  for (int th = 1; th <= 3; th += 2) {
    double* sf2 = (double*)calloc((size_t)nh * dk * dv, sizeof(double));
    efla_oracle_fwd(0, q, k, v, beta, s0, o, sf, NULL, nh, T, dk, dv, 1);
    if (efla_oracle_fwd_gated(0, q, k, v, beta, z, s0, o, sf2, nh, T, dk, dv, th) != 0) ++fails;
    for (long e = 0; e < nh * dk * dv; ++e)
      if (fabs(sf2[e] - sf[e]) > 1e-9 * (1.0 + fabs(sf[e]))) ++fails;
    free(sf2);
  }
  if (efla_oracle_fwd_gated(0, q, k, v, beta, NULL, s0, o, sf, nh, T, dk, dv, 1) != -1) ++fails;
  /* one step on one head, no output */
  double S[24];
  memcpy(S, s0, sizeof(S));
  efla_oracle_step(0, q, k, v, 0.5, S, NULL, dk, dv);
  efla_oracle_step_gated(0, q, k, v, 0.5, -0.3, S, NULL, dk, dv);
  free(z), free(q), free(k), free(v), free(beta), free(s0), free(dout), free(dsT), free(o), free(sf), free(sn);
  printf("oracle sanitizer driver: %d failed checks\n", fails);
  return fails ? 1 : 0;
}
