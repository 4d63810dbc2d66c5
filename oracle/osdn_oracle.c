/*
 * OSDN forward oracle: the plain token-by-token recurrence in fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Tests, the smoke check and the benchmark's
 * CPU-baseline leg may call it; the GPU library never does, and the two share
 * no code.  It is deliberately slow and obvious: no blocking, no fusion, no
 * reordering beyond the definition.
 *
 * Source of every formula: the gist.science technical summary of
 * "OSDN: Improving Delta Rule with Provable Online Preconditioning in Linear
 * Attention" (arXiv 2605.13473), cited below as [summary §N], and the arXiv
 * abstract of the same paper, cited as [abstract].
 *
 * Per (batch b, head h), with S in R^{dv x dk} stored row-major [dv][dk]:
 *
 *   d <- d0 (default all ones)           S <- S0 (default zero)
 *   for t = 0 .. T-1:
 *     n   = ||k_t||^2,  a = <d, k_t (.) k_t>          [summary §2.2, terms of h_t]
 *     kt  = d (.) k_t                                 [summary §2.1, preconditioned key]
 *     u   = v_t - S k_t                               [summary §1, residual of f_t at S_{t-1}]
 *     S  += beta_t u kt^T                             [summary §2.1, update with kt]
 *     o_t = S q_t                                     readout after the write (a stated choice;
 *                                                     the pages define no readout)
 *     rho = (1 - beta_t a)^2                          [summary §3, token-local residual ratio]
 *     g   = -beta_t (1 - beta_t a) k_t(.)k_t / n      gradient in d of the closed-form
 *                                                     surrogate [summary §2.2]; 0 when n = 0
 *     d   = r_t d - eta g                             [summary §2.3, APF; r_t = 1 without APF;
 *                                                     descent, as OGD in §2.2 requires]
 *
 * Modes: OSDN (above), DELTANET (kt = k_t, d unused: the plain delta rule of
 * [summary §1]) and GIVEN_KTILDE (kt read from an input; isolates the state
 * pass).  In every mode rho_t = (1 - beta_t <kt, k_t>)^2, which equals the
 * OSDN formula because <d (.) k, k> = <d, k (.) k>.
 *
 * Optional state gate alpha_t (Gated DeltaNet backbone, [summary §4] lists it
 * among the evaluated backbones but prints no formula; the plainest reading):
 * the state decays before the token's read and write,
 *     S <- alpha_t S,  then u = v_t - S k_t and S += beta_t u kt^T as above,
 * i.e. S_t = alpha_t S_{t-1} + beta_t (v_t - alpha_t S_{t-1} k_t) kt^T.  The
 * preconditioner walk and rho_t do not involve S and are unchanged.  NULL
 * alpha is alpha = 1.
 *
 * Optional per-channel gate alpha_k (Kimi Delta Attention backbone, also only
 * named in [summary §4]; the plainest reading generalises the scalar gate to
 * one gate per key dimension): each column i of S (key dimension i) decays by
 * alpha_k[t][i] before the token's read and write,
 *     S <- S diag(alpha_k_t),  then u = v_t - S k_t and S += beta_t u kt^T,
 * i.e. S_t = S_{t-1} D_t + beta_t (v_t - S_{t-1} D_t k_t) kt^T, D_t = diag(alpha_k_t).
 * A gate vector with equal entries is the scalar gate.
 */
#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_OSDN = 0, ORACLE_DELTANET = 1, ORACLE_GIVEN_KTILDE = 2 };

typedef struct {
  int B, H, T, dk, dv, mode;
  double eta;
  const double *q, *k, *v, *beta, *r, *d0, *S0, *k_given, *alpha, *alpha_k;
  double *o, *S_final, *d_final, *k_tilde, *d_all, *rho;
  const long *heads; /* which flattened (b,h) indices to run */
  long n_heads;
  long next;         /* work counter, protected by lock */
  pthread_mutex_t lock;
  int failed;
} oracle_job;

/* One (b,h) sequence.  All arrays are indexed with the flattened head bh. */
static int run_head(const oracle_job *J, long bh) {
  const int T = J->T, dk = J->dk, dv = J->dv;
  double *S = (double *)malloc(sizeof(double) * (size_t)dv * dk);
  double *d = (double *)malloc(sizeof(double) * (size_t)dk);
  double *kt = (double *)malloc(sizeof(double) * (size_t)dk);
  double *u = (double *)malloc(sizeof(double) * (size_t)dv);
  if (!S || !d || !kt || !u) {
    free(S); free(d); free(kt); free(u);
    return -1;
  }
  if (J->S0) memcpy(S, J->S0 + bh * (long)dv * dk, sizeof(double) * (size_t)dv * dk);
  else memset(S, 0, sizeof(double) * (size_t)dv * dk);
  for (int i = 0; i < dk; ++i) d[i] = J->d0 ? J->d0[bh * dk + i] : 1.0;

  for (int t = 0; t < T; ++t) {
    const long row = bh * (long)T + t;
    const double *k = J->k + row * dk;
    const double *v = J->v + row * dv;
    const double beta = J->beta[row];
    const double rt = J->r ? J->r[row] : 1.0;

    /* key statistics */
    double n = 0.0, a = 0.0;
    for (int i = 0; i < dk; ++i) {
      const double p = k[i] * k[i];
      n += p;
      a += d[i] * p;
    }

    /* write key */
    if (J->mode == ORACLE_OSDN) {
      for (int i = 0; i < dk; ++i) kt[i] = d[i] * k[i];
    } else if (J->mode == ORACLE_DELTANET) {
      for (int i = 0; i < dk; ++i) kt[i] = k[i];
    } else {
      const double *kg = J->k_given + row * dk;
      for (int i = 0; i < dk; ++i) kt[i] = kg[i];
    }
    if (J->k_tilde) memcpy(J->k_tilde + row * dk, kt, sizeof(double) * (size_t)dk);
    if (J->d_all) memcpy(J->d_all + row * dk, d, sizeof(double) * (size_t)dk);

    /* state gate: the decay acts before the token's read and write */
    if (J->alpha) {
      const double at = J->alpha[row];
      for (long x = 0; x < (long)dv * dk; ++x) S[x] *= at;
    }
    if (J->alpha_k) {
      const double *ak = J->alpha_k + row * dk;
      for (int j = 0; j < dv; ++j)
        for (int i = 0; i < dk; ++i) S[(long)j * dk + i] *= ak[i];
    }

    /* residual against the state before this token's write */
    for (int j = 0; j < dv; ++j) {
      double sk = 0.0;
      for (int i = 0; i < dk; ++i) sk += S[(long)j * dk + i] * k[i];
      u[j] = v[j] - sk;
    }

    /* delta-rule write with the (preconditioned) key */
    for (int j = 0; j < dv; ++j)
      for (int i = 0; i < dk; ++i) S[(long)j * dk + i] += beta * u[j] * kt[i];

    /* readout with the state after the write */
    if (J->o) {
      const double *q = J->q + row * dk;
      for (int j = 0; j < dv; ++j) {
        double s = 0.0;
        for (int i = 0; i < dk; ++i) s += S[(long)j * dk + i] * q[i];
        J->o[row * dv + j] = s;
      }
    }

    /* token-local residual ratio */
    double kk = a;
    if (J->mode != ORACLE_OSDN) {
      kk = 0.0;
      for (int i = 0; i < dk; ++i) kk += kt[i] * k[i];
    }
    if (J->rho) J->rho[row] = (1.0 - beta * kk) * (1.0 - beta * kk);

    /* preconditioner step: descent on the closed-form surrogate, then APF retention */
    if (J->mode == ORACLE_OSDN) {
      for (int i = 0; i < dk; ++i) {
        const double grad = (n > 0.0) ? -beta * (1.0 - beta * a) * (k[i] * k[i]) / n : 0.0;
        d[i] = rt * d[i] - J->eta * grad;
      }
    }
  }

  if (J->S_final) memcpy(J->S_final + bh * (long)dv * dk, S, sizeof(double) * (size_t)dv * dk);
  if (J->d_final) memcpy(J->d_final + bh * dk, d, sizeof(double) * (size_t)dk);
  free(S); free(d); free(kt); free(u);
  return 0;
}

static void *worker(void *arg) {
  oracle_job *J = (oracle_job *)arg;
  for (;;) {
    pthread_mutex_lock(&J->lock);
    const long idx = J->next++;
    pthread_mutex_unlock(&J->lock);
    if (idx >= J->n_heads) break;
    const long bh = J->heads ? J->heads[idx] : idx;
    if (run_head(J, bh) != 0) {
      pthread_mutex_lock(&J->lock);
      J->failed = 1;
      pthread_mutex_unlock(&J->lock);
    }
  }
  return NULL;
}

/*
 * Run the recurrence over the heads listed in `heads` (flattened b*H+h; NULL
 * means all B*H heads) with up to n_threads threads (one head per task).
 * Shapes: q,k,k_given,k_tilde,d_all [B,H,T,dk]; v,o [B,H,T,dv];
 * beta,r,alpha,rho [B,H,T]; alpha_k [B,H,T,dk]; d0,d_final [B,H,dk];
 * S0,S_final [B,H,dv,dk].
 * Optional pointers may be NULL.  Returns 0, or -1 on bad arguments or
 * allocation failure.
 */
int oracle_forward(int B, int H, int T, int dk, int dv, int mode, double eta,
                   const double *q, const double *k, const double *v,
                   const double *beta, const double *r, const double *d0,
                   const double *S0, const double *k_given, const double *alpha,
                   const double *alpha_k, double *o, double *S_final, double *d_final,
                   double *k_tilde, double *d_all, double *rho,
                   const long *heads, long n_heads, int n_threads) {
  if (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0) return -1;
  if (mode < ORACLE_OSDN || mode > ORACLE_GIVEN_KTILDE) return -1;
  if (T > 0 && (!k || !v || !beta)) return -1;
  if (o && T > 0 && !q) return -1;
  if (mode == ORACLE_GIVEN_KTILDE && T > 0 && !k_given) return -1;
  if (!heads) n_heads = (long)B * H;
  if (n_threads < 1) n_threads = 1;
  if (n_threads > n_heads) n_threads = n_heads > 0 ? (int)n_heads : 1;

  oracle_job J;
  memset(&J, 0, sizeof(J));
  J.B = B; J.H = H; J.T = T; J.dk = dk; J.dv = dv; J.mode = mode; J.eta = eta;
  J.q = q; J.k = k; J.v = v; J.beta = beta; J.r = r; J.d0 = d0; J.S0 = S0;
  J.k_given = k_given; J.alpha = alpha; J.alpha_k = alpha_k; J.o = o; J.S_final = S_final; J.d_final = d_final;
  J.k_tilde = k_tilde; J.d_all = d_all; J.rho = rho;
  J.heads = heads; J.n_heads = n_heads; J.next = 0; J.failed = 0;
  pthread_mutex_init(&J.lock, NULL);

  if (n_threads == 1) {
    worker(&J);
  } else {
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
    int started = 0;
    if (th) {
      for (; started < n_threads; ++started)
        if (pthread_create(&th[started], NULL, worker, &J) != 0) break;
    }
    if (started == 0) worker(&J);
    for (int i = 0; i < started; ++i) pthread_join(th[i], NULL);
    free(th);
  }
  pthread_mutex_destroy(&J.lock);
  return J.failed ? -1 : 0;
}
