/*
 * KDA oracle: plain, slow, obviously-correct fp64 CPU reference.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. The product path (the
 * HIP library and its Python binding) never calls into it and shares no code,
 * header or constant with it.
 *
 * Sources (web pages, cited by title and section):
 *   [KDA-blog]  "Kimi k3 技术报告详解（1）——架构再升华" (stevenstage.github.io,
 *               posts/blog7), sections "Kimi Delta Attention" and
 *               "Chunkwise parallel form".
 *   [Baidu-1]   "Kimi K3 Core Techniques Explained: How Three Innovations
 *               Reshape LLM Training Efficiency", §1.2 Mechanism Design.
 *   [Baidu-2]   "A Look at Kimi K3: Three Core Innovations and Engineering
 *               Tuning Guide", §2.2 (the kda_decay pseudocode).
 *
 * What is computed:
 *   kda_oracle_gate        g = g_min * sigmoid(exp(A_h) * z)
 *                          [KDA-blog §Chunkwise parallel form, new-gate
 *                          equation; Baidu-2 §2.2 kda_decay]
 *   kda_oracle_cumsum      chunk-local inclusive cumulative sum of g, i.e.
 *                          log gamma^r = sum_{i<=r} log alpha^i, restarting at
 *                          each sequence start and every C tokens from it
 *                          [KDA-blog §Chunkwise parallel form, gamma equation]
 *   kda_oracle_recurrence  the KDA recurrence, one token at a time
 *                          S_t = (I - b_t k_t k_t^T) Diag(alpha_t) S_{t-1}
 *                                + b_t k_t v_t^T,   o_t = S_t^T q_t
 *                          [KDA-blog §Kimi Delta Attention, KDA equation]
 *                          with alpha_t = exp(g_t) [KDA-blog, new-gate
 *                          equation]. No chunking: the chunkwise form is
 *                          stated on the same page to equal this exactly.
 *
 * Parity pins (closed forms, invariants, brute force) live in the tests.
 * Build: gcc -O2 -std=c99 -shared -fPIC (no fast-math, no intrinsics).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ gate */

/* Logistic function in fp64, written so that it never overflows. */
static double sigmoid(double x) {
  if (x >= 0.0) return 1.0 / (1.0 + exp(-x));
  double e = exp(x);
  return e / (1.0 + e);
}

/*
 * g[i] = g_min * sigmoid(exp(A[h]) * z[i]) for a tensor laid out as
 * [rows, H, Dk] (rows = B*T). A may be NULL, meaning A_h = 0 (exp(A_h) = 1).
 * [KDA-blog §Chunkwise parallel form, new-gate equation]
 */
void kda_oracle_gate(const double* z, const double* A, double g_min, long rows,
                     int H, int Dk, double* g) {
  for (long r = 0; r < rows; ++r)
    for (int h = 0; h < H; ++h) {
      double scale = A ? exp(A[h]) : 1.0;
      for (int c = 0; c < Dk; ++c) {
        long i = (r * H + h) * (long)Dk + c;
        g[i] = g_min * sigmoid(scale * z[i]);
      }
    }
}

/*
 * Chunk-local inclusive cumsum over the token axis of a packed tensor
 * [Ttot, H, Dk]. Sequence n spans tokens [cu[n], cu[n+1]); chunks of `chunk`
 * tokens start at cu[n]. Inclusive: element r holds g_1 + ... + g_r of its
 * chunk, matching gamma^r = prod_{i=1}^{r} alpha^i.
 * [KDA-blog §Chunkwise parallel form, gamma equation]
 */
void kda_oracle_cumsum(const double* g, const int32_t* cu, int N, int H, int Dk,
                       int chunk, double* out) {
  for (int n = 0; n < N; ++n)
    for (int h = 0; h < H; ++h)
      for (int c = 0; c < Dk; ++c) {
        double run = 0.0;
        for (long t = cu[n]; t < cu[n + 1]; ++t) {
          if ((t - cu[n]) % chunk == 0) run = 0.0;
          long i = (t * H + h) * (long)Dk + c;
          run += g[i];
          out[i] = run;
        }
      }
}

/* ------------------------------------------------------------ recurrence */

/*
 * One (sequence, head) unit, token by token, in fp64.
 *   S      [Dk][Dv], in: initial state, out: final state
 *   q,k,g  rows of Dk values, token t at base + t*stride
 *   v,o    rows of Dv values
 *   beta   one value per token, token t at beta[t*beta_stride]
 * Per token [KDA-blog §Kimi Delta Attention, KDA equation]:
 *   1. S <- Diag(alpha) S             alpha = exp(g_t)
 *   2. u <- S^T k                      the value currently stored under k
 *   3. d <- beta (v - u)               delta-rule correction
 *   4. S <- S + k d^T                  rank-1 write
 *   5. o <- scale * S^T q              read after the write (o_t uses S_t)
 * Steps 1-4 expand to (I - beta k k^T) Diag(alpha) S + beta k v^T.
 */
static void unit_recurrence(long T, int Dk, int Dv, const double* q, const double* k,
                            const double* v, const double* g, long row_stride_k,
                            long row_stride_v, const double* beta, long beta_stride,
                            double scale, double* S, double* o) {
  double* u = (double*)malloc(sizeof(double) * (size_t)Dv);
  for (long t = 0; t < T; ++t) {
    const double* qt = q + t * row_stride_k;
    const double* kt = k + t * row_stride_k;
    const double* gt = g + t * row_stride_k;
    const double* vt = v + t * row_stride_v;
    double bt = beta[t * beta_stride];
    /* 1. decay each row i of S by alpha_i */
    for (int i = 0; i < Dk; ++i) {
      double a = exp(gt[i]);
      for (int j = 0; j < Dv; ++j) S[i * Dv + j] *= a;
    }
    /* 2. u = S^T k */
    for (int j = 0; j < Dv; ++j) u[j] = 0.0;
    for (int i = 0; i < Dk; ++i)
      for (int j = 0; j < Dv; ++j) u[j] += S[i * Dv + j] * kt[i];
    /* 3. d = beta (v - u), kept in u */
    for (int j = 0; j < Dv; ++j) u[j] = bt * (vt[j] - u[j]);
    /* 4. S += k d^T */
    for (int i = 0; i < Dk; ++i)
      for (int j = 0; j < Dv; ++j) S[i * Dv + j] += kt[i] * u[j];
    /* 5. o = scale * S^T q */
    double* ot = o + t * row_stride_v;
    for (int j = 0; j < Dv; ++j) ot[j] = 0.0;
    for (int i = 0; i < Dk; ++i)
      for (int j = 0; j < Dv; ++j) ot[j] += S[i * Dv + j] * qt[i];
    for (int j = 0; j < Dv; ++j) ot[j] *= scale;
  }
  free(u);
}

typedef struct {
  int H, Dk, Dv;
  const double *q, *k, *v, *g, *beta, *h0;
  const int32_t* cu;
  double scale;
  double *o, *hT;
  const int32_t* order; /* units (n*H + h), longest sequence first */
  int n_units;
  int next; /* shared work counter */
  pthread_mutex_t lock;
} job_t;

static void run_unit(job_t* jb, int unit) {
  int H = jb->H, Dk = jb->Dk, Dv = jb->Dv;
  int n = unit / H, h = unit % H;
  long t0 = jb->cu[n], T = (long)jb->cu[n + 1] - t0;
  size_t ssz = (size_t)Dk * Dv;
  double* S = jb->hT + (size_t)unit * ssz;
  if (jb->h0)
    memcpy(S, jb->h0 + (size_t)unit * ssz, sizeof(double) * ssz);
  else
    memset(S, 0, sizeof(double) * ssz);
  long rk = (long)H * Dk, rv = (long)H * Dv;
  unit_recurrence(T, Dk, Dv, jb->q + t0 * rk + (long)h * Dk, jb->k + t0 * rk + (long)h * Dk,
                  jb->v + t0 * rv + (long)h * Dv, jb->g + t0 * rk + (long)h * Dk, rk, rv,
                  jb->beta + t0 * H + h, H, jb->scale, S, jb->o + t0 * rv + (long)h * Dv);
}

static void* worker(void* arg) {
  job_t* jb = (job_t*)arg;
  for (;;) {
    pthread_mutex_lock(&jb->lock);
    int i = jb->next++;
    pthread_mutex_unlock(&jb->lock);
    if (i >= jb->n_units) break;
    run_unit(jb, jb->order[i]);
  }
  return NULL;
}

typedef struct {
  long len;
  int32_t unit;
} unit_len_t;

static int by_length_desc(const void* a, const void* b) {
  const unit_len_t* x = (const unit_len_t*)a;
  const unit_len_t* y = (const unit_len_t*)b;
  if (x->len != y->len) return x->len > y->len ? -1 : 1;
  return x->unit - y->unit;
}

/*
 * Packed layout: q, k, g [Ttot, H, Dk]; v, o [Ttot, H, Dv]; beta [Ttot, H];
 * h0, hT [N, H, Dk, Dv] (h0 may be NULL = zeros). Sequence n covers tokens
 * [cu[n], cu[n+1]); a dense batch of B sequences of length T is cu = {0, T,
 * 2T, ...}. Units (sequence, head) are independent and run on `nthreads`
 * threads, longest first. g is the per-token log-decay (alpha = exp(g)).
 * Returns 0, or -1 on bad arguments.
 */
int kda_oracle_recurrence(const double* q, const double* k, const double* v, const double* g,
                          const double* beta, const double* h0, const int32_t* cu, int N,
                          int H, int Dk, int Dv, double scale, double* o, double* hT,
                          int nthreads) {
  if (!q || !k || !v || !g || !beta || !cu || !o || !hT || N < 0 || H <= 0 || Dk <= 0 ||
      Dv <= 0)
    return -1;
  for (int n = 0; n < N; ++n)
    if (cu[n + 1] < cu[n]) return -1;
  job_t jb;
  jb.H = H; jb.Dk = Dk; jb.Dv = Dv;
  jb.q = q; jb.k = k; jb.v = v; jb.g = g; jb.beta = beta; jb.h0 = h0;
  jb.cu = cu; jb.scale = scale; jb.o = o; jb.hT = hT;
  jb.n_units = N * H;
  jb.next = 0;
  size_t nu = (size_t)(jb.n_units > 0 ? jb.n_units : 1);
  unit_len_t* ul = (unit_len_t*)malloc(sizeof(unit_len_t) * nu);
  int32_t* order = (int32_t*)malloc(sizeof(int32_t) * nu);
  for (int i = 0; i < jb.n_units; ++i) {
    ul[i].unit = i;
    ul[i].len = (long)cu[i / H + 1] - cu[i / H];
  }
  qsort(ul, (size_t)jb.n_units, sizeof(unit_len_t), by_length_desc);
  for (int i = 0; i < jb.n_units; ++i) order[i] = ul[i].unit;
  free(ul);
  jb.order = order;
  pthread_mutex_init(&jb.lock, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > jb.n_units) nthreads = jb.n_units > 0 ? jb.n_units : 1;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, &jb);
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&jb.lock);
  free(order);
  return 0;
}
