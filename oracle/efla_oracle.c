/*
 * EFLA reference oracle — TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, sequential fp64 CPU implementation of the Exact Flow Linear
 * Attention recurrence. Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load this library; the product path never does. It shares
 * no code, header or constant with the GPU library.
 *
 * What it computes (papernotes.org note "Exact Flow Linear Attention: Exact
 * Solution from Continuous-Time Dynamics", section 关键设计, items 1-2, and the
 * flowchart of section 整体框架):
 *
 *   lambda_t = k_t . k_t                      (the only nonzero eigenvalue of k k^T)
 *   alpha_t  = (1 - exp(-beta_t*lambda_t)) / lambda_t
 *   S_t      = (I - alpha_t k_t k_t^T) S_{t-1} + alpha_t k_t v_t^T
 *   o_t      = S_t^T q_t                      (read out after the update)
 *
 * Numerics follow the same note, section 损失函数 / 训练策略: the denominator is
 * floored at 1e-12 and the numerator is formed as -expm1(-beta*lambda), never
 * as 1 - exp(...). The floored lambda is used in both places (the plain reading
 * that keeps alpha -> beta as lambda -> 0, section 关键设计 item 3).
 *
 * The state S is d_k x d_v, row index = key dimension (the write k v^T fixes
 * that orientation). Heads are independent; each is run token by token.
 *
 * The same rank-1 step also runs with three other coefficients (one scalar c
 * in place of alpha; everything else unchanged):
 *   - explicit Euler, c = beta: the delta rule the note contrasts with
 *     (关键设计 item 1);
 *   - one-step RK4 (jsqmd.com article "EFLA注意力机制：优化挑战与训练策略解析",
 *     section 5.3): the printed matrix polynomial in A = k k^T collapses,
 *     because A^n = lambda^(n-1) A, to c = beta (1 - x/2 + x^2/6 - x^3/24)
 *     with x = beta lambda, for both the transition and the input term;
 *   - second order (same section names it without writing it out; the plain
 *     reading is the same series cut after the A^2 term):
 *     c = beta (1 - x/2).
 * No floor applies to lambda in these three: none of them divides by it.
 * Also exposed, for tests only: the Frobenius norm of the state after every
 * step; and a gated variant (efla_oracle_step_gated / efla_oracle_fwd_gated),
 * the reading taken of the pages' "Gated EFLA": the same step applied to the
 * state decayed by a per-token factor g_t = exp(log_g_t).
 *
 * Parity pins live in the test suite (the gated variant's in
 * test_oracle_gated_pins.py): the worked example printed in the note
 * (section 一个完整示例), scipy's matrix exponential of the augmented ODE
 * matrix, a fine-step RK4 integration of dS/dt = -k k^T S + k v^T, a truncated
 * Taylor series with scaling and squaring, mpmath alpha, limits, bounds,
 * invariants and an independent chunked (WY/UT) evaluation.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#define EFLA_ORACLE_EXACT 0
#define EFLA_ORACLE_EULER 1
#define EFLA_ORACLE_RK4 2
#define EFLA_ORACLE_ORDER2 3

/* Exact-flow coefficient with the 1e-12 floor on lambda (training-strategy
 * section of the papernotes note; rank-1 collapse in 关键设计 item 2). */
double efla_oracle_alpha(double beta, double lam) {
  double lamc = lam > 1e-12 ? lam : 1e-12;
  return -expm1(-beta * lamc) / lamc;
}

/* The scalar of the rank-1 step for each mode (see the header comment). */
double efla_oracle_coef(int mode, double beta, double lam) {
  double x = beta * lam;
  switch (mode) {
    case EFLA_ORACLE_EULER: return beta;
    case EFLA_ORACLE_RK4: return beta * (1.0 - x / 2.0 + x * x / 6.0 - x * x * x / 24.0);
    case EFLA_ORACLE_ORDER2: return beta * (1.0 - x / 2.0);
    default: return efla_oracle_alpha(beta, lam);
  }
}

/* One token on one head. S is d_k x d_v row-major, updated in place.
 * o (length d_v) receives S_t^T q after the update. */
void efla_oracle_step(int mode, const double* q, const double* k, const double* v,
                      double beta, double* S, double* o, int dk, int dv) {
  double lam = 0.0;
  for (int i = 0; i < dk; ++i) lam += k[i] * k[i];
  double a = efla_oracle_coef(mode, beta, lam);

  /* p = S^T k, then S <- S - a k p^T + a k v^T  ==  (I - a k k^T) S + a k v^T */
  double* p = (double*)malloc(sizeof(double) * (size_t)dv);
  for (int j = 0; j < dv; ++j) p[j] = 0.0;
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) p[j] += k[i] * S[(size_t)i * dv + j];
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) S[(size_t)i * dv + j] += a * k[i] * (v[j] - p[j]);
  free(p);

  if (o) {
    for (int j = 0; j < dv; ++j) {
      double acc = 0.0;
      for (int i = 0; i < dk; ++i) acc += S[(size_t)i * dv + j] * q[i];
      o[j] = acc;
    }
  }
}

/* Gated EFLA, one token on one head. The pages name a gated variant (the
 * papernotes note's main-results table, "Gated EFLA", and its key findings:
 * the exact flow upgrades Gated DeltaNet) but print no formula. The reading
 * taken here: Gated DeltaNet's update with its step coefficient replaced by
 * the exact-flow one,
 *   S_t = g_t (I - c k k^T) S_{t-1} + c k v^T,   g_t = exp(log_g),
 * i.e. the ungated step applied to the decayed state g_t S_{t-1}; with
 * log_g = 0 it is the step above. Steps in that order: lambda and c, p = S^T k,
 * S <- g (S - c k p^T) + c k v^T, o = S^T q. */
void efla_oracle_step_gated(int mode, const double* q, const double* k, const double* v,
                            double beta, double log_g, double* S, double* o, int dk, int dv) {
  double lam = 0.0;
  for (int i = 0; i < dk; ++i) lam += k[i] * k[i];
  double a = efla_oracle_coef(mode, beta, lam);
  double g = exp(log_g);

  double* p = (double*)malloc(sizeof(double) * (size_t)dv);
  for (int j = 0; j < dv; ++j) p[j] = 0.0;
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) p[j] += k[i] * S[(size_t)i * dv + j];
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j)
      S[(size_t)i * dv + j] = g * (S[(size_t)i * dv + j] - a * k[i] * p[j]) + a * k[i] * v[j];
  free(p);

  if (o) {
    for (int j = 0; j < dv; ++j) {
      double acc = 0.0;
      for (int i = 0; i < dk; ++i) acc += S[(size_t)i * dv + j] * q[i];
      o[j] = acc;
    }
  }
}

typedef struct {
  int mode;
  const double *q, *k, *v, *beta, *s0;
  double *o, *s_final, *snorm;
  const double* log_g; /* [nh, T] log-decays (gated variant), or NULL */
  long nh, T;
  int dk, dv;
  long h_begin, h_end;
} oracle_job;

static void run_head(const oracle_job* J, long h) {
  const long T = J->T;
  const int dk = J->dk, dv = J->dv;
  const size_t ss = (size_t)dk * dv;
  double* S = (double*)malloc(sizeof(double) * ss);
  if (J->s0) memcpy(S, J->s0 + (size_t)h * ss, sizeof(double) * ss);
  else memset(S, 0, sizeof(double) * ss);

  for (long t = 0; t < T; ++t) {
    const double* q = J->q + ((size_t)h * T + t) * dk;
    const double* k = J->k + ((size_t)h * T + t) * dk;
    const double* v = J->v + ((size_t)h * T + t) * dv;
    double b = J->beta[(size_t)h * T + t];
    double* o = J->o ? J->o + ((size_t)h * T + t) * dv : NULL;
    if (J->log_g)
      efla_oracle_step_gated(J->mode, q, k, v, b, J->log_g[(size_t)h * T + t], S, o, dk, dv);
    else
      efla_oracle_step(J->mode, q, k, v, b, S, o, dk, dv);
    if (J->snorm) {
      double n2 = 0.0;
      for (size_t e = 0; e < ss; ++e) n2 += S[e] * S[e];
      J->snorm[(size_t)h * T + t] = sqrt(n2);
    }
  }
  if (J->s_final) memcpy(J->s_final + (size_t)h * ss, S, sizeof(double) * ss);
  free(S);
}

static void* run_range(void* arg) {
  const oracle_job* J = (const oracle_job*)arg;
  for (long h = J->h_begin; h < J->h_end; ++h) run_head(J, h);
  return NULL;
}

/*
 * Sequential forward over nh independent heads.
 *   q, k  [nh, T, dk]    v [nh, T, dv]    beta [nh, T]
 *   s0    [nh, dk, dv] or NULL (zeros)
 *   o     [nh, T, dv] or NULL          (out)
 *   s_final [nh, dk, dv] or NULL       (out)
 *   snorm [nh, T] or NULL              (out: ||S_t||_F after each token)
 * nthreads <= 1 runs on the calling thread. Returns 0, or -1 on bad sizes.
 */
static int run_heads(oracle_job base, int nthreads) {
  const long nh = base.nh;
  if (nh < 0 || base.T < 0 || base.dk < 1 || base.dv < 1) return -1;
  if (nh == 0) return 0;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > nh) nthreads = (int)nh;
  if (nthreads == 1) {
    run_range(&base);
    return 0;
  }
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  oracle_job* jobs = (oracle_job*)malloc(sizeof(oracle_job) * (size_t)nthreads);
  long per = nh / nthreads, rem = nh % nthreads, h = 0;
  for (int i = 0; i < nthreads; ++i) {
    jobs[i] = base;
    jobs[i].h_begin = h;
    h += per + (i < rem ? 1 : 0);
    jobs[i].h_end = h;
    pthread_create(&th[i], NULL, run_range, &jobs[i]);
  }
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(th);
  free(jobs);
  return 0;
}

int efla_oracle_fwd(int mode, const double* q, const double* k, const double* v,
                    const double* beta, const double* s0, double* o, double* s_final,
                    double* snorm, long nh, long T, int dk, int dv, int nthreads) {
  oracle_job base = {mode, q, k, v, beta, s0, o, s_final, snorm, NULL, nh, T, dk, dv, 0, nh};
  return run_heads(base, nthreads);
}

/* The gated variant over nh heads: as efla_oracle_fwd, with log_g [nh, T]
 * the per-token log-decays (efla_oracle_step_gated). */
int efla_oracle_fwd_gated(int mode, const double* q, const double* k, const double* v,
                          const double* beta, const double* log_g, const double* s0, double* o,
                          double* s_final, long nh, long T, int dk, int dv, int nthreads) {
  if (!log_g) return -1;
  oracle_job base = {mode, q, k, v, beta, s0, o, s_final, NULL, log_g, nh, T, dk, dv, 0, nh};
  return run_heads(base, nthreads);
}

/* ---------------------------------------------------------------------------
 * Backward (reverse mode through the token-serial forward above). The pages
 * give no gradient formulas: this is the derivative of the forward as it
 * stands, written step by step. With u_t = c_t (v_t - S_{t-1}^T k_t),
 * S_t = S_{t-1} + k_t u_t^T, o_t = S_t^T q_t, and G_t the gradient of the
 * loss with respect to S_t (starting from the given dS_T), walking t down:
 *   G    += q_t do_t^T,        dq_t  = S_t do_t
 *   du    = G^T k_t,           dk_t  = G u_t - c_t S_{t-1} du
 *   dv_t  = c_t du,            dc_t  = du . (v_t - S_{t-1}^T k_t)
 *   G_{t-1} = G - c_t k_t du^T
 * and the scalar's chain rule: dbeta_t = dc_t dc/dbeta, dk_t += 2 dc_t
 * (dc/dlambda) k_t.
 */

/* dc/dbeta and dc/dlambda of efla_oracle_coef. */
void efla_oracle_coef_grad(int mode, double beta, double lam, double* dbeta, double* dlam) {
  double x = beta * lam;
  switch (mode) {
    case EFLA_ORACLE_EULER:
      *dbeta = 1.0;
      *dlam = 0.0;
      return;
    case EFLA_ORACLE_RK4:
      *dbeta = 1.0 - x + x * x / 2.0 - x * x * x / 6.0;
      *dlam = beta * beta * (-0.5 + x / 3.0 - x * x / 8.0);
      return;
    case EFLA_ORACLE_ORDER2:
      *dbeta = 1.0 - x;
      *dlam = -beta * beta / 2.0;
      return;
    default: {
      double lamc = lam > 1e-12 ? lam : 1e-12;
      double xc = beta * lamc;
      *dbeta = exp(-xc);
      if (!(lam > 1e-12)) {
        *dlam = 0.0; /* the floor makes the coefficient constant in lambda */
      } else if (fabs(xc) < 1e-3) {
        /* (beta e^{-x} - c)/lambda = beta^2 sum_{n>=1} (-1)^n n x^{n-1}/(n+1)! */
        *dlam = beta * beta * (-0.5 + xc / 3.0 - xc * xc / 8.0 + xc * xc * xc / 30.0);
      } else {
        *dlam = (beta * exp(-xc) - efla_oracle_alpha(beta, lam)) / lamc;
      }
    }
  }
}

typedef struct {
  int mode;
  const double *q, *k, *v, *beta, *s0, *dout, *dsT;
  double *dq, *dk, *dv, *dbeta, *ds0;
  long nh, T;
  int dk_, dv_;
  long h_begin, h_end;
} oracle_bwd_job;

static void bwd_head(const oracle_bwd_job* J, long h) {
  const long T = J->T;
  const int dk = J->dk_, dv = J->dv_;
  const size_t ss = (size_t)dk * dv;
  /* every state S_0..S_T of the forward */
  double* St = (double*)malloc(sizeof(double) * ss * (size_t)(T + 1));
  if (J->s0) memcpy(St, J->s0 + (size_t)h * ss, sizeof(double) * ss);
  else memset(St, 0, sizeof(double) * ss);
  for (long t = 0; t < T; ++t) {
    memcpy(St + (size_t)(t + 1) * ss, St + (size_t)t * ss, sizeof(double) * ss);
    efla_oracle_step(J->mode, J->q + ((size_t)h * T + t) * dk, J->k + ((size_t)h * T + t) * dk,
                     J->v + ((size_t)h * T + t) * dv, J->beta[(size_t)h * T + t],
                     St + (size_t)(t + 1) * ss, NULL, dk, dv);
  }
  double* G = (double*)malloc(sizeof(double) * ss);
  if (J->dsT) memcpy(G, J->dsT + (size_t)h * ss, sizeof(double) * ss);
  else memset(G, 0, sizeof(double) * ss);
  double* du = (double*)malloc(sizeof(double) * (size_t)dv);
  double* u = (double*)malloc(sizeof(double) * (size_t)dv);
  double* p = (double*)malloc(sizeof(double) * (size_t)dv);
  for (long t = T - 1; t >= 0; --t) {
    const double* q = J->q + ((size_t)h * T + t) * dk;
    const double* k = J->k + ((size_t)h * T + t) * dk;
    const double* v = J->v + ((size_t)h * T + t) * dv;
    const double* dout = J->dout + ((size_t)h * T + t) * dv;
    double* dq = J->dq + ((size_t)h * T + t) * dk;
    double* dkk = J->dk + ((size_t)h * T + t) * dk;
    double* dvv = J->dv + ((size_t)h * T + t) * dv;
    const double* Sp = St + (size_t)t * ss;       /* S_{t-1} */
    const double* Sn = St + (size_t)(t + 1) * ss; /* S_t */
    const double b = J->beta[(size_t)h * T + t];
    double lam = 0.0;
    for (int i = 0; i < dk; ++i) lam += k[i] * k[i];
    const double c = efla_oracle_coef(J->mode, b, lam);
    /* read-out of S_t */
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) G[(size_t)i * dv + j] += q[i] * dout[j];
    for (int i = 0; i < dk; ++i) {
      double acc = 0.0;
      for (int j = 0; j < dv; ++j) acc += Sn[(size_t)i * dv + j] * dout[j];
      dq[i] = acc;
    }
    /* u = c (v - S_{t-1}^T k) */
    for (int j = 0; j < dv; ++j) {
      double acc = 0.0;
      for (int i = 0; i < dk; ++i) acc += Sp[(size_t)i * dv + j] * k[i];
      p[j] = v[j] - acc;
      u[j] = c * p[j];
    }
    double dc = 0.0;
    for (int j = 0; j < dv; ++j) {
      double acc = 0.0;
      for (int i = 0; i < dk; ++i) acc += G[(size_t)i * dv + j] * k[i];
      du[j] = acc;
      dvv[j] = c * acc;
      dc += acc * p[j];
    }
    for (int i = 0; i < dk; ++i) {
      double a1 = 0.0, a2 = 0.0;
      for (int j = 0; j < dv; ++j) {
        a1 += G[(size_t)i * dv + j] * u[j];
        a2 += Sp[(size_t)i * dv + j] * du[j];
      }
      dkk[i] = a1 - c * a2;
    }
    double gb, gl;
    efla_oracle_coef_grad(J->mode, b, lam, &gb, &gl);
    J->dbeta[(size_t)h * T + t] = dc * gb;
    for (int i = 0; i < dk; ++i) dkk[i] += 2.0 * dc * gl * k[i];
    /* G_{t-1} = G - c k du^T */
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) G[(size_t)i * dv + j] -= c * k[i] * du[j];
  }
  if (J->ds0) memcpy(J->ds0 + (size_t)h * ss, G, sizeof(double) * ss);
  free(St);
  free(G);
  free(du);
  free(u);
  free(p);
}

static void* bwd_range(void* arg) {
  const oracle_bwd_job* J = (const oracle_bwd_job*)arg;
  for (long h = J->h_begin; h < J->h_end; ++h) bwd_head(J, h);
  return NULL;
}

/*
 * Gradients of a loss L(o, S_T) given dout = dL/do [nh, T, dv] and dsT =
 * dL/dS_T [nh, dk, dv] (NULL: zero). Outputs dq, dk [nh, T, dk], dv [nh, T, dv],
 * dbeta [nh, T], ds0 [nh, dk, dv] (NULL: not written). s0 NULL means zeros.
 * Returns 0, or -1 on bad sizes.
 */
int efla_oracle_bwd(int mode, const double* q, const double* k, const double* v,
                    const double* beta, const double* s0, const double* dout, const double* dsT,
                    double* dq, double* dk, double* dv, double* dbeta, double* ds0, long nh, long T,
                    int dk_, int dv_, int nthreads) {
  if (nh < 0 || T < 0 || dk_ < 1 || dv_ < 1) return -1;
  if (nh == 0) return 0;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > nh) nthreads = (int)nh;
  oracle_bwd_job base = {mode, q, k, v, beta, s0, dout, dsT, dq, dk, dv, dbeta, ds0,
                         nh, T, dk_, dv_, 0, nh};
  if (nthreads == 1) {
    bwd_range(&base);
    return 0;
  }
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  oracle_bwd_job* jobs = (oracle_bwd_job*)malloc(sizeof(oracle_bwd_job) * (size_t)nthreads);
  long per = nh / nthreads, rem = nh % nthreads, h = 0;
  for (int i = 0; i < nthreads; ++i) {
    jobs[i] = base;
    jobs[i].h_begin = h;
    h += per + (i < rem ? 1 : 0);
    jobs[i].h_end = h;
    pthread_create(&th[i], NULL, bwd_range, &jobs[i]);
  }
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(th);
  free(jobs);
  return 0;
}
