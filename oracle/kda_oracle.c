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
 *   kda_oracle_gate_bwd    derivative of the gate w.r.t. z and A_h
 *   kda_oracle_backward    derivative of the recurrence w.r.t. q, k, v, g,
 *                          beta and the initial state, given the gradients
 *                          of every o_t and of the final state: each forward
 *                          step differentiated in reverse order, from states
 *                          kept by a forward pass. The pages do not give a
 *                          backward; this is the plain derivative.
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

/* -------------------------------------------------------------- backward */

/*
 * Gradient of the gate g = g_min * sigmoid(s z), s = exp(A_h), for a tensor
 * laid out as [rows, H, Dk]: with p = sigmoid(s z) and p' = p (1 - p),
 *   dz = dg * g_min * p' * s,     dA_h = sum over rows, c of dg * g_min * p' * s * z.
 * dA may be NULL (not wanted); A may be NULL (A_h = 0).
 * [KDA-blog §Chunkwise parallel form, new-gate equation], differentiated.
 */
void kda_oracle_gate_bwd(const double* z, const double* A, double g_min, const double* dg,
                         long rows, int H, int Dk, double* dz, double* dA) {
  if (dA)
    for (int h = 0; h < H; ++h) dA[h] = 0.0;
  for (long r = 0; r < rows; ++r)
    for (int h = 0; h < H; ++h) {
      double s = A ? exp(A[h]) : 1.0;
      for (int c = 0; c < Dk; ++c) {
        long i = (r * H + h) * (long)Dk + c;
        double p = sigmoid(s * z[i]);
        double dx = dg[i] * g_min * p * (1.0 - p); /* gradient w.r.t. x = s z */
        dz[i] = dx * s;
        if (dA) dA[h] += dx * s * z[i];
      }
    }
}

/*
 * Reverse-mode derivative of unit_recurrence for one unit: given do (the
 * gradient of the loss w.r.t. every o_t) and dS (w.r.t. the final state, in:
 * [Dk][Dv], out: the gradient w.r.t. the initial state), writes the
 * gradients w.r.t. q, k, v, g and beta. The pages state the forward
 * recurrence only [KDA-blog §Kimi Delta Attention, KDA equation]; this is
 * its exact derivative, every step of the forward undone in reverse order
 * (Sb = the decayed state, u = Sb^T k, d = beta (v - u)):
 *   5. o = scale S^T q         dq = scale S do;           dS += scale q do^T
 *   4. S = Sb + k d^T          dd = dS^T k;  dk = dS d;   dSb = dS
 *   3. d = beta (v - u)        dv = beta dd; dbeta = dd . (v - u); du = -beta dd
 *   2. u = Sb^T k              dSb += k du^T;  dk += Sb du
 *   1. Sb = Diag(alpha) S_prev dg_i = sum_j dSb_ij Sb_ij;  dS_prev = Diag(alpha) dSb
 * The states S_0 .. S_T of the forward pass are kept (T+1 of them).
 * Returns 0, or -1 if memory runs out.
 */
static int unit_backward(long T, int Dk, int Dv, const double* q, const double* k,
                         const double* v, const double* g, long rk, long rv, const double* beta,
                         long bs, double scale, const double* h0, const double* dO, double* dS,
                         double* dq, double* dk, double* dv, double* dg, double* dbeta) {
  size_t ssz = (size_t)Dk * Dv;
  double* st = (double*)malloc(sizeof(double) * ssz * (size_t)(T + 1));
  double* Sb = (double*)malloc(sizeof(double) * ssz);
  double* u = (double*)malloc(sizeof(double) * (size_t)Dv * 3);
  if (!st || !Sb || !u) {
    free(st); free(Sb); free(u);
    return -1;
  }
  double* d = u + Dv;
  double* dd = u + 2 * Dv;
  /* forward pass, keeping every state */
  if (h0)
    memcpy(st, h0, sizeof(double) * ssz);
  else
    memset(st, 0, sizeof(double) * ssz);
  for (long t = 0; t < T; ++t) {
    const double *kt = k + t * rk, *gt = g + t * rk, *vt = v + t * rv;
    double bt = beta[t * bs];
    double* S = st + (size_t)(t + 1) * ssz;
    for (int i = 0; i < Dk; ++i) {
      double al = exp(gt[i]);
      for (int j = 0; j < Dv; ++j) S[i * Dv + j] = al * st[(size_t)t * ssz + i * Dv + j];
    }
    for (int j = 0; j < Dv; ++j) u[j] = 0.0;
    for (int i = 0; i < Dk; ++i)
      for (int j = 0; j < Dv; ++j) u[j] += kt[i] * S[i * Dv + j];
    for (int j = 0; j < Dv; ++j) d[j] = bt * (vt[j] - u[j]);
    for (int i = 0; i < Dk; ++i)
      for (int j = 0; j < Dv; ++j) S[i * Dv + j] += kt[i] * d[j];
  }
  /* reverse pass */
  for (long t = T - 1; t >= 0; --t) {
    const double *qt = q + t * rk, *kt = k + t * rk, *gt = g + t * rk, *vt = v + t * rv;
    const double* dot = dO + t * rv;
    double bt = beta[t * bs];
    const double* S = st + (size_t)(t + 1) * ssz;
    const double* Sp = st + (size_t)t * ssz;
    double *dqt = dq + t * rk, *dkt = dk + t * rk, *dgt = dg + t * rk, *dvt = dv + t * rv;
    /* 5. o = scale S^T q */
    for (int i = 0; i < Dk; ++i) {
      double acc = 0.0;
      for (int j = 0; j < Dv; ++j) acc += S[i * Dv + j] * dot[j];
      dqt[i] = scale * acc;
      for (int j = 0; j < Dv; ++j) dS[i * Dv + j] += scale * qt[i] * dot[j];
    }
    /* recompute the decayed state, u and d of this token */
    for (int i = 0; i < Dk; ++i) {
      double al = exp(gt[i]);
      for (int j = 0; j < Dv; ++j) Sb[i * Dv + j] = al * Sp[i * Dv + j];
    }
    for (int j = 0; j < Dv; ++j) u[j] = 0.0;
    for (int i = 0; i < Dk; ++i)
      for (int j = 0; j < Dv; ++j) u[j] += kt[i] * Sb[i * Dv + j];
    for (int j = 0; j < Dv; ++j) d[j] = bt * (vt[j] - u[j]);
    /* 4. S = Sb + k d^T */
    for (int j = 0; j < Dv; ++j) dd[j] = 0.0;
    for (int i = 0; i < Dk; ++i) {
      double acc = 0.0;
      for (int j = 0; j < Dv; ++j) {
        dd[j] += dS[i * Dv + j] * kt[i];
        acc += dS[i * Dv + j] * d[j];
      }
      dkt[i] = acc;
    }
    /* 3. d = beta (v - u); du = -beta dd is kept in dd */
    double db = 0.0;
    for (int j = 0; j < Dv; ++j) {
      dvt[j] = bt * dd[j];
      db += dd[j] * (vt[j] - u[j]);
      dd[j] = -bt * dd[j];
    }
    dbeta[t * bs] = db;
    /* 2. u = Sb^T k */
    for (int i = 0; i < Dk; ++i) {
      double acc = 0.0;
      for (int j = 0; j < Dv; ++j) {
        dS[i * Dv + j] += kt[i] * dd[j];
        acc += Sb[i * Dv + j] * dd[j];
      }
      dkt[i] += acc;
    }
    /* 1. Sb = Diag(alpha) S_prev */
    for (int i = 0; i < Dk; ++i) {
      double al = exp(gt[i]), acc = 0.0;
      for (int j = 0; j < Dv; ++j) {
        acc += dS[i * Dv + j] * Sb[i * Dv + j];
        dS[i * Dv + j] *= al;
      }
      dgt[i] = acc;
    }
  }
  free(st); free(Sb); free(u);
  return 0;
}

typedef struct {
  int H, Dk, Dv;
  const double *q, *k, *v, *g, *beta, *h0, *dO, *dhT;
  const int32_t* cu;
  double scale;
  double *dq, *dk, *dv, *dg, *dbeta, *dh0;
  int n_units;
  int next, failed;
  pthread_mutex_t lock;
} bjob_t;

static void* bworker(void* arg) {
  bjob_t* jb = (bjob_t*)arg;
  for (;;) {
    pthread_mutex_lock(&jb->lock);
    int unit = jb->next++;
    pthread_mutex_unlock(&jb->lock);
    if (unit >= jb->n_units) break;
    int H = jb->H, Dk = jb->Dk, Dv = jb->Dv;
    int n = unit / H, h = unit % H;
    long t0 = jb->cu[n], T = (long)jb->cu[n + 1] - t0;
    size_t ssz = (size_t)Dk * Dv;
    double* dS = jb->dh0 + (size_t)unit * ssz;
    if (jb->dhT)
      memcpy(dS, jb->dhT + (size_t)unit * ssz, sizeof(double) * ssz);
    else
      memset(dS, 0, sizeof(double) * ssz);
    long rk = (long)H * Dk, rv = (long)H * Dv;
    long ok = t0 * rk + (long)h * Dk, ov = t0 * rv + (long)h * Dv, ob = t0 * H + h;
    int rc = unit_backward(T, Dk, Dv, jb->q + ok, jb->k + ok, jb->v + ov, jb->g + ok, rk, rv,
                           jb->beta + ob, H, jb->scale, jb->h0 ? jb->h0 + (size_t)unit * ssz : NULL,
                           jb->dO + ov, dS, jb->dq + ok, jb->dk + ok, jb->dv + ov, jb->dg + ok,
                           jb->dbeta + ob);
    if (rc) {
      pthread_mutex_lock(&jb->lock);
      jb->failed = 1;
      pthread_mutex_unlock(&jb->lock);
    }
  }
  return NULL;
}

/*
 * Backward of kda_oracle_recurrence, same packed layout: dO like o, dhT like
 * hT (NULL = zero gradient on the final state); writes dq, dk, dg like q,
 * dv like v, dbeta like beta and dh0 like h0. Units run on `nthreads`
 * threads; each keeps T+1 states of Dk*Dv doubles. Returns 0, or -1 on bad
 * arguments or when memory runs out.
 */
int kda_oracle_backward(const double* q, const double* k, const double* v, const double* g,
                        const double* beta, const double* h0, const int32_t* cu, int N, int H,
                        int Dk, int Dv, double scale, const double* dO, const double* dhT,
                        double* dq, double* dk, double* dv, double* dg, double* dbeta,
                        double* dh0, int nthreads) {
  if (!q || !k || !v || !g || !beta || !cu || !dO || !dq || !dk || !dv || !dg || !dbeta ||
      !dh0 || N < 0 || H <= 0 || Dk <= 0 || Dv <= 0)
    return -1;
  for (int n = 0; n < N; ++n)
    if (cu[n + 1] < cu[n]) return -1;
  bjob_t jb;
  jb.H = H; jb.Dk = Dk; jb.Dv = Dv;
  jb.q = q; jb.k = k; jb.v = v; jb.g = g; jb.beta = beta; jb.h0 = h0; jb.dO = dO; jb.dhT = dhT;
  jb.cu = cu; jb.scale = scale;
  jb.dq = dq; jb.dk = dk; jb.dv = dv; jb.dg = dg; jb.dbeta = dbeta; jb.dh0 = dh0;
  jb.n_units = N * H;
  jb.next = 0;
  jb.failed = 0;
  pthread_mutex_init(&jb.lock, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > jb.n_units) nthreads = jb.n_units > 0 ? jb.n_units : 1;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nthreads);
  for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, bworker, &jb);
  for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  free(th);
  pthread_mutex_destroy(&jb.lock);
  return jb.failed ? -1 : 0;
}
