/*
 * Plain fp64 CPU oracle for the Gaussian Mixture Attention (GMA) forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the parity reference for the HIP
 * library; only the test suite, the smoke check and the benchmark's CPU
 * baseline may build, load or call it.  It shares no code, header or table
 * with the HIP path.
 *
 * Source: "Gaussian Mixture Attention: Linear-Time Sequence Mixing via
 * Probabilistic Latent Routing" (arXiv 2606.18283, HTML version), Section
 * "Gaussian routing components" (Eqs. 2-3), "Projections" (Eq. 4), "Latent
 * aggregation / normalized broadcasting" (Eqs. 5-7 and footnote 4), "Causal
 * GMA" (Eq. 8b and footnote 6), "Learning" (Eq. 15) and "Gradient structure"
 * (Eq. 16, responsibilities as a softmax of scores).
 *
 * Everything is computed in double precision with straight loops in the
 * order the definitions give; the only parallelism is over independent
 * (batch, head) units.  Where the extracted text lost an equation the reading
 * taken is stated next to the code.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define GMAO_LOG_2PI 1.8378770664093454835606594728112

/* Eq. 15: pi = softmax(alpha).  Returns log pi_k = alpha_k - log sum_l exp(alpha_l).
 * The library's log_pi argument may carry any per-head additive constant; the
 * oracle normalises it here so that pi sums to one exactly as in the text. */
static void log_prior(const double* alpha, int K, double* logpi) {
  double m = alpha[0];
  for (int k = 1; k < K; ++k) if (alpha[k] > m) m = alpha[k];
  double s = 0.0;
  for (int k = 0; k < K; ++k) s += exp(alpha[k] - m);
  double lse = m + log(s);
  for (int k = 0; k < K; ++k) logpi[k] = alpha[k] - lse;
}

/* Eqs. 2-3 (display equations lost in extraction; the surviving prose and
 * Eq. 16 define them): the joint log-probability of routing vector x and
 * component k under a GMM with diagonal covariance,
 *   s_k = log pi_k + log N(x; mu_k, diag(sigma^2_k))
 *       = log pi_k - 1/2 sum_d [ (x_d - mu_kd)^2 / sigma^2_kd + log sigma^2_kd + log 2pi ].
 * The covariance diagonal is given as log sigma^2. */
static void scores(const double* x, int d_r, const double* mu, const double* ls2,
                   const double* logpi, int K, double* s) {
  for (int k = 0; k < K; ++k) {
    double q = 0.0;
    for (int d = 0; d < d_r; ++d) {
      double diff = x[d] - mu[(size_t)k * d_r + d];
      double var = exp(ls2[(size_t)k * d_r + d]);
      q += diff * diff / var + ls2[(size_t)k * d_r + d] + GMAO_LOG_2PI;
    }
    s[k] = logpi[k] - 0.5 * q;
  }
}

/* Eq. 3 / Eq. 16: gamma_k = exp(s_k) / sum_l exp(s_l), evaluated with the
 * maximum subtracted.  Hard assignment z = argmax_k gamma_k, ties to the
 * lowest index. */
static int32_t posterior(const double* s, int K, double* gamma) {
  int32_t arg = 0;
  double m = s[0];
  for (int k = 1; k < K; ++k)
    if (s[k] > m) { m = s[k]; arg = k; }
  double tot = 0.0;
  for (int k = 0; k < K; ++k) { gamma[k] = exp(s[k] - m); tot += gamma[k]; }
  for (int k = 0; k < K; ++k) gamma[k] /= tot;
  return arg;
}

typedef struct {
  const double *Q, *Kx, *V, *mu, *ls2, *alpha;
  int64_t B, H, N;
  int d_r, d_v, K;
  double eps;
  int causal;
  const int64_t* rows;   /* sorted ascending, or NULL for all rows */
  int64_t nrows;
  double* out;           /* [B,H,nout,d_v] */
  int32_t* assign_q;     /* [B,H,nout] or NULL */
  int32_t* assign_k;     /* [B,H,N] or NULL */
  double* vtilde;        /* [B,H,K,d_v] or NULL (bidirectional only) */
  double* ztot;          /* [B,H,K] or NULL (bidirectional only) */
  int64_t next_unit;
  pthread_mutex_t lock;
} fwd_job;

static void forward_unit(fwd_job* j, int64_t u) {
  const int64_t h = u % j->H;
  const int d_r = j->d_r, d_v = j->d_v, K = j->K;
  const int64_t N = j->N;
  const int64_t nout = j->rows ? j->nrows : N;
  const double* q = j->Q + (size_t)u * N * d_r;
  const double* kx = j->Kx + (size_t)u * N * d_r;
  const double* v = j->V + (size_t)u * N * d_v;
  const double* mu = j->mu + (size_t)h * K * d_r;
  const double* ls2 = j->ls2 + (size_t)h * K * d_r;
  double* o = j->out + (size_t)u * nout * d_v;

  double* logpi = malloc(sizeof(double) * K);
  double* s = malloc(sizeof(double) * K);
  double* gk = malloc(sizeof(double) * K);
  double* gq = malloc(sizeof(double) * K);
  double* vt = calloc((size_t)K * d_v, sizeof(double));   /* V~ (or its prefix) */
  double* z = calloc((size_t)K, sizeof(double));          /* Z  (or its prefix) */
  log_prior(j->alpha + (size_t)h * K, K, logpi);

  if (!j->causal) {
    /* Eqs. 5-6: V~_k = sum_j gamma^K_jk v_j,  Z_k = sum_j gamma^K_jk. */
    for (int64_t t = 0; t < N; ++t) {
      scores(kx + (size_t)t * d_r, d_r, mu, ls2, logpi, K, s);
      int32_t a = posterior(s, K, gk);
      if (j->assign_k) j->assign_k[(size_t)u * N + t] = a;
      for (int k = 0; k < K; ++k) {
        z[k] += gk[k];
        for (int e = 0; e < d_v; ++e) vt[(size_t)k * d_v + e] += gk[k] * v[(size_t)t * d_v + e];
      }
    }
    if (j->vtilde) memcpy(j->vtilde + (size_t)u * K * d_v, vt, sizeof(double) * K * d_v);
    if (j->ztot) memcpy(j->ztot + (size_t)u * K, z, sizeof(double) * K);
    /* Eq. 7: O_i = gamma^Q_i V~ / (gamma^Q_i . Z + eps). */
    for (int64_t r = 0; r < nout; ++r) {
      int64_t i = j->rows ? j->rows[r] : r;
      scores(q + (size_t)i * d_r, d_r, mu, ls2, logpi, K, s);
      int32_t a = posterior(s, K, gq);
      if (j->assign_q) j->assign_q[(size_t)u * nout + r] = a;
      double den = 0.0;
      for (int k = 0; k < K; ++k) den += gq[k] * z[k];
      den += j->eps;
      for (int e = 0; e < d_v; ++e) {
        double num = 0.0;
        for (int k = 0; k < K; ++k) num += gq[k] * vt[(size_t)k * d_v + e];
        o[(size_t)r * d_v + e] = num / den;
      }
    }
  } else {
    /* Causal GMA: prefix memories V~^(i)_k = sum_{j<=i} gamma^K_jk v_j and
     * Z^(i)_k = sum_{j<=i} gamma^K_jk (inclusive prefix, "positions j <= i"),
     * O_i = gamma^Q_i V~^(i) / (gamma^Q_i . Z^(i) + eps), the row-wise form of
     * Eq. 8b with the same stabiliser as Eq. 7.  A plain running sum. */
    int64_t r = 0;
    for (int64_t i = 0; i < N; ++i) {
      scores(kx + (size_t)i * d_r, d_r, mu, ls2, logpi, K, s);
      int32_t a = posterior(s, K, gk);
      if (j->assign_k) j->assign_k[(size_t)u * N + i] = a;
      for (int k = 0; k < K; ++k) {
        z[k] += gk[k];
        for (int e = 0; e < d_v; ++e) vt[(size_t)k * d_v + e] += gk[k] * v[(size_t)i * d_v + e];
      }
      int want = j->rows ? (r < nout && j->rows[r] == i) : 1;
      if (!want) continue;
      scores(q + (size_t)i * d_r, d_r, mu, ls2, logpi, K, s);
      int32_t aq = posterior(s, K, gq);
      if (j->assign_q) j->assign_q[(size_t)u * nout + r] = aq;
      double den = 0.0;
      for (int k = 0; k < K; ++k) den += gq[k] * z[k];
      den += j->eps;
      for (int e = 0; e < d_v; ++e) {
        double num = 0.0;
        for (int k = 0; k < K; ++k) num += gq[k] * vt[(size_t)k * d_v + e];
        o[(size_t)r * d_v + e] = num / den;
      }
      ++r;
      if (j->rows && r >= nout) break;
    }
  }
  free(logpi); free(s); free(gk); free(gq); free(vt); free(z);
}

static void* forward_worker(void* arg) {
  fwd_job* j = (fwd_job*)arg;
  for (;;) {
    pthread_mutex_lock(&j->lock);
    int64_t u = j->next_unit++;
    pthread_mutex_unlock(&j->lock);
    if (u >= j->B * j->H) break;
    forward_unit(j, u);
  }
  return NULL;
}

/* Full GMA forward over a [B,H,N,*] batch.  Parameters are per head:
 * mu, ls2 [H,K,d_r], alpha [H,K].  If rows != NULL only the listed output rows
 * (sorted ascending) are produced, in that order; the memories are still built
 * from every key as the definitions require.  Returns 0 on success. */
int gmao_forward(const double* Q, const double* Kx, const double* V,
                 const double* mu, const double* ls2, const double* alpha,
                 int64_t B, int64_t H, int64_t N, int d_r, int d_v, int K,
                 double eps, int causal, const int64_t* rows, int64_t nrows,
                 double* out, int32_t* assign_q, int32_t* assign_k,
                 double* vtilde, double* ztot, int nthreads) {
  if (B < 1 || H < 1 || N < 1 || d_r < 1 || d_v < 1 || K < 1) return 1;
  if (rows) {
    for (int64_t r = 0; r < nrows; ++r) {
      if (rows[r] < 0 || rows[r] >= N) return 2;
      if (r > 0 && rows[r] <= rows[r - 1]) return 3;
    }
  }
  fwd_job j = {Q, Kx, V, mu, ls2, alpha, B, H, N, d_r, d_v, K, eps, causal,
               rows, nrows, out, assign_q, assign_k, vtilde, ztot, 0};
  pthread_mutex_init(&j.lock, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  for (int t = 0; t < nthreads; ++t) pthread_create(&th[t], NULL, forward_worker, &j);
  for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
  pthread_mutex_destroy(&j.lock);
  return 0;
}

/* Responsibilities alone (Eq. 3) for U units of N routing vectors each; unit u
 * uses the parameters of head (u % H).  gamma [U,N,K] (may be NULL),
 * assign [U,N] (may be NULL), score [U,N,K] natural-log scores (may be NULL). */
int gmao_resp(const double* X, int64_t U, int64_t H, int64_t N, int d_r,
              const double* mu, const double* ls2, const double* alpha, int K,
              double* gamma, int32_t* assign, double* score) {
  if (U < 1 || H < 1 || N < 1 || d_r < 1 || K < 1) return 1;
  double* logpi = malloc(sizeof(double) * K);
  double* s = malloc(sizeof(double) * K);
  double* g = malloc(sizeof(double) * K);
  for (int64_t u = 0; u < U; ++u) {
    int64_t h = u % H;
    log_prior(alpha + (size_t)h * K, K, logpi);
    for (int64_t i = 0; i < N; ++i) {
      scores(X + ((size_t)u * N + i) * d_r, d_r, mu + (size_t)h * K * d_r,
             ls2 + (size_t)h * K * d_r, logpi, K, s);
      int32_t a = posterior(s, K, g);
      size_t off = ((size_t)u * N + i) * K;
      if (gamma) memcpy(gamma + off, g, sizeof(double) * K);
      if (score) memcpy(score + off, s, sizeof(double) * K);
      if (assign) assign[(size_t)u * N + i] = a;
    }
  }
  free(logpi); free(s); free(g);
  return 0;
}
