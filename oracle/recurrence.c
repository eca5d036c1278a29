/*
 * TEST INFRASTRUCTURE ONLY -- the fp64 CPU oracle for delta-rule linear
 * attention.  Only tests, the smoke check and the benchmark's CPU-baseline
 * leg may load this; the product path never does.
 *
 * What it computes: the plain token-by-token recurrence of a delta-rule
 * linear-attention head, as "Empowering Hybrid Attention Models on NPUs"
 * describes it in Section 2.1 ("Architecture of Linear-Attention Hybrids"):
 * at step t the state S_{t-1} is updated with K_t and V_t, then the output
 * is read from the updated state with Q_t.  The update itself (the gated
 * delta rule of GDN, and its per-channel-gated form KDA, both named in
 * Section 1 and Section 2.1) is written here with the state stored
 * key-major, S in R^{dk x dv}:
 *
 *   GDN:  S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T,  a_t = exp(g_t)
 *   KDA:  S_t = (I - b_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + b_t k_t v_t^T
 *   both: o_t = S_t^T q_t
 *
 * evaluated in the order: decay S; x = S^T k; S += b k (v - x)^T;
 * o = S^T q.  No chunking, blocking or reordering.
 *
 * Layouts (all row-major, token-major, packed over sequences):
 *   q, k  [T, h_qk, dk]; v, o [T, h_v, dv]; beta [T, h_v];
 *   g [T, h_v] (GDN) or [T, h_v, dk] (KDA); h0, ht [N, h_v, dk, dv].
 * v-head h reads q/k head h / (h_v / h_qk).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int kda, n_seqs, h_qk, h_v, dk, dv;
  const int64_t* cu;
  const double *q, *k, *v, *beta, *g, *h0;
  double *o, *ht;
  int n_units;
  int next; /* guarded by lock */
  pthread_mutex_t lock;
} job_t;

static void run_unit(const job_t* J, int unit, double* S, double* x) {
  const int seq = unit / J->h_v, h = unit % J->h_v;
  const int grp = J->h_v / J->h_qk, hk = h / grp;
  const int dk = J->dk, dv = J->dv;
  const size_t sidx = ((size_t)seq * J->h_v + h) * (size_t)dk * dv;
  if (J->h0)
    memcpy(S, J->h0 + sidx, sizeof(double) * dk * dv);
  else
    memset(S, 0, sizeof(double) * dk * dv);
  for (int64_t t = J->cu[seq]; t < J->cu[seq + 1]; ++t) {
    const double* qt = J->q + ((size_t)t * J->h_qk + hk) * dk;
    const double* kt = J->k + ((size_t)t * J->h_qk + hk) * dk;
    const double* vt = J->v + ((size_t)t * J->h_v + h) * dv;
    const double bt = J->beta[(size_t)t * J->h_v + h];
    /* decay */
    if (J->kda) {
      const double* gt = J->g + ((size_t)t * J->h_v + h) * dk;
      for (int i = 0; i < dk; ++i) {
        const double a = exp(gt[i]);
        for (int j = 0; j < dv; ++j) S[i * dv + j] *= a;
      }
    } else {
      const double a = exp(J->g[(size_t)t * J->h_v + h]);
      for (int i = 0; i < dk * dv; ++i) S[i] *= a;
    }
    /* x = S^T k */
    for (int j = 0; j < dv; ++j) x[j] = 0.0;
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) x[j] += S[i * dv + j] * kt[i];
    /* S += beta k (v - x)^T */
    for (int j = 0; j < dv; ++j) x[j] = bt * (vt[j] - x[j]);
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) S[i * dv + j] += kt[i] * x[j];
    /* o = S^T q */
    double* ot = J->o + ((size_t)t * J->h_v + h) * dv;
    for (int j = 0; j < dv; ++j) ot[j] = 0.0;
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) ot[j] += S[i * dv + j] * qt[i];
  }
  if (J->ht) memcpy(J->ht + sidx, S, sizeof(double) * dk * dv);
}

static void* worker(void* arg) {
  job_t* J = (job_t*)arg;
  double* S = (double*)malloc(sizeof(double) * (size_t)J->dk * J->dv);
  double* x = (double*)malloc(sizeof(double) * (size_t)J->dv);
  for (;;) {
    pthread_mutex_lock(&J->lock);
    const int u = J->next++;
    pthread_mutex_unlock(&J->lock);
    if (u >= J->n_units) break;
    run_unit(J, u, S, x);
  }
  free(S);
  free(x);
  return NULL;
}

/* Returns 0 on success, -1 on a malformed argument. */
int oracle_delta_rule_f64(int kda, int n_seqs, const int64_t* cu_seqlens,
                          int h_qk, int h_v, int dk, int dv,
                          const double* q, const double* k, const double* v,
                          const double* beta, const double* g,
                          const double* h0, double* o, double* ht,
                          int n_threads) {
  if (n_seqs < 0 || h_qk <= 0 || h_v <= 0 || dk <= 0 || dv <= 0) return -1;
  if (h_v % h_qk != 0) return -1;
  if (!cu_seqlens || !q || !k || !v || !beta || !g || !o) return -1;
  for (int s = 0; s < n_seqs; ++s)
    if (cu_seqlens[s + 1] < cu_seqlens[s]) return -1;
  job_t J;
  J.kda = kda; J.n_seqs = n_seqs; J.h_qk = h_qk; J.h_v = h_v;
  J.dk = dk; J.dv = dv; J.cu = cu_seqlens;
  J.q = q; J.k = k; J.v = v; J.beta = beta; J.g = g; J.h0 = h0;
  J.o = o; J.ht = ht;
  J.n_units = n_seqs * h_v;
  J.next = 0;
  pthread_mutex_init(&J.lock, NULL);
  if (n_threads < 1) n_threads = 1;
  if (n_threads > J.n_units) n_threads = J.n_units > 0 ? J.n_units : 1;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * n_threads);
  for (int i = 1; i < n_threads; ++i) pthread_create(&th[i], NULL, worker, &J);
  worker(&J);
  for (int i = 1; i < n_threads; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&J.lock);
  return 0;
}

/*
 * Decay-only linear attention (no delta rule): the temporal-decay form of
 * RetNet and GLA that "Empowering Hybrid Attention Models on NPUs" names in
 * Section 8 (Related Work) beside GDN and KDA.  Same layouts, no beta:
 *
 *   scalar gate      S_t = exp(g_t) S_{t-1} + k_t v_t^T
 *   per-channel gate S_t = Diag(exp(g_t)) S_{t-1} + k_t v_t^T
 *   both:            o_t = S_t^T q_t
 *
 * evaluated in the order: decay S; S += k v^T; o = S^T q.
 */
typedef struct {
  int per_channel, n_seqs, h_qk, h_v, dk, dv;
  const int64_t* cu;
  const double *q, *k, *v, *g, *h0;
  double *o, *ht;
} decay_job_t;

static void run_decay_unit(const decay_job_t* J, int unit, double* S) {
  const int seq = unit / J->h_v, h = unit % J->h_v;
  const int hk = h / (J->h_v / J->h_qk);
  const int dk = J->dk, dv = J->dv;
  const size_t sidx = ((size_t)seq * J->h_v + h) * (size_t)dk * dv;
  if (J->h0)
    memcpy(S, J->h0 + sidx, sizeof(double) * dk * dv);
  else
    memset(S, 0, sizeof(double) * dk * dv);
  for (int64_t t = J->cu[seq]; t < J->cu[seq + 1]; ++t) {
    const double* qt = J->q + ((size_t)t * J->h_qk + hk) * dk;
    const double* kt = J->k + ((size_t)t * J->h_qk + hk) * dk;
    const double* vt = J->v + ((size_t)t * J->h_v + h) * dv;
    for (int i = 0; i < dk; ++i) {
      const double a = J->per_channel ? exp(J->g[((size_t)t * J->h_v + h) * dk + i])
                                      : exp(J->g[(size_t)t * J->h_v + h]);
      for (int j = 0; j < dv; ++j) S[i * dv + j] = a * S[i * dv + j] + kt[i] * vt[j];
    }
    double* ot = J->o + ((size_t)t * J->h_v + h) * dv;
    for (int j = 0; j < dv; ++j) ot[j] = 0.0;
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) ot[j] += S[i * dv + j] * qt[i];
  }
  if (J->ht) memcpy(J->ht + sidx, S, sizeof(double) * dk * dv);
}

/* Single-threaded (test sizes).  Returns 0 on success, -1 on a malformed
 * argument. */
int oracle_decay_f64(int per_channel, int n_seqs, const int64_t* cu_seqlens,
                     int h_qk, int h_v, int dk, int dv,
                     const double* q, const double* k, const double* v,
                     const double* g, const double* h0, double* o, double* ht) {
  if (n_seqs < 0 || h_qk <= 0 || h_v <= 0 || dk <= 0 || dv <= 0) return -1;
  if (h_v % h_qk != 0) return -1;
  if (!cu_seqlens || !q || !k || !v || !g || !o) return -1;
  for (int s = 0; s < n_seqs; ++s)
    if (cu_seqlens[s + 1] < cu_seqlens[s]) return -1;
  decay_job_t J = {per_channel, n_seqs, h_qk, h_v, dk, dv, cu_seqlens, q, k, v, g, h0, o, ht};
  double* S = (double*)malloc(sizeof(double) * (size_t)dk * dv);
  for (int u = 0; u < n_seqs * h_v; ++u) run_decay_unit(&J, u, S);
  free(S);
  return 0;
}
