/*
 * pic_oracle.c -- plain fp64 CPU oracle for the linear-attention segment
 * transform of position-independent caching (HYPIC).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The product
 * path (the HIP library) never links, calls or includes anything here, and
 * this file shares no code, header, table or constant with it.
 *
 * What it computes, and where the pages state it:
 *
 *  - A linear-attention layer keeps one recurrent state per head,
 *    S in R^{dk x dv}.  Each token applies a linear transition T_t to the
 *    incoming state and adds its own write term:
 *        S_t = T_t * S_{t-1} + beta_t * k_t * v_t^T.
 *    [xix.ai HYPIC article (French), paragraph on linear layers:
 *     transition matrices of tokens; families RetNet, Mamba2, GLA,
 *     DeltaNet, GDN, KDA.  remio.ai HYPIC article (Japanese), section
 *     "HYPICが線形アテンション状態を合成する仕組み": scalar, diagonal and
 *     dense transition forms.]
 *
 *    The per-token transition of each family (the pages name the families
 *    but print no formula; the plainest reading of each family):
 *        scalar decay   T_t = alpha_t * I              (beta = 1)
 *        diagonal gate  T_t = Diag(alpha_t)            (beta = 1)
 *        dense GDN      T_t = alpha_t * (I - beta_t k_t k_t^T)
 *        dense KDA      T_t = (I - beta_t k_t k_t^T) Diag(alpha_t)
 *
 *  - A segment C = tokens [o, o+L) started from the zero state yields the
 *    pair (T_C, S(C|0)): T_C is the product of all token transitions of the
 *    segment, latest on the left, and S(C|0) is the final state.
 *    [xix.ai, paragraph on linear layers: the accumulated transition
 *     operator T_C and the zero-start state S(C|0) depend only on the
 *     segment's own tokens.]
 *
 *  - Reuse composes pairs: S(C1.C2) = T(C2) * S(C1) + S(C2), i.e. the
 *    running state is left-multiplied by T_C and S(C|0) is added.
 *    [xix.ai, paragraph on linear layers, the composition identity.]
 *
 *  - The naive ablation adds zero-start states and drops T:
 *    S_in + sum_i S(C_i|0).
 *    [xix.ai, paragraph on linear layers: simple addition of zero-start
 *     final states, valid only for plain linear attention;
 *     remio.ai (Japanese), same section: naive addition cannot reproduce
 *     the sequential state.]
 *
 *  - Reuse with seam windows: the first tokens of an inner segment are
 *    kept out of its cached pair and, on reuse, run from the running state
 *    one by one, each emitting its output o_t = S_t^T q_t, before the pair
 *    of the rest of the segment is applied (oracle_seam_compose, below).
 *    [xix.ai, paragraph on full-attention layers: seam windows of w tokens.]
 *
 *  - Prefill with outputs: a segment prefilled on its own (from the zero
 *    state) also gives every token's output o_t = S_t^T q_t, read from the
 *    state right after the token's update (oracle_prefill, below): the
 *    computation in which the pair is built at first prefill.
 *    [remio.ai (Japanese), same section: the pair is cached at the
 *     segment's first prefill, a small add-on to it.]
 *
 *  Because T_C underflows fp32 at realistic gate values, the pair is also
 *  given in split form: lambda_C = sum_t ln(alpha_t) (per head for scalar
 *  and dense, per key channel for diagonal) and, for the dense form,
 *  That_C = prod_t (I - beta_t k_t k_t^T), so that T_C = e^{lambda_C}*That_C.
 *  For the KDA form the gate does not factor out of the product; lambda_C =
 *  sum_t ln m_t with m_t the token's largest gate, and That_C is the product
 *  of (I - beta_t k_t k_t^T) Diag(alpha_t / m_t): the same split when all
 *  channels share one gate, and That_C stays bounded (norm <= 1).
 *  The oracle computes both factors directly (not by dividing T_C).
 *
 *  Two build paths are offered:
 *    literal      -- forms each T_t as an explicit dense dk x dk matrix and
 *                    applies it with explicit matrix products (O(dk^3) per
 *                    token); this is the definition written out.
 *    specialised  -- the same definition with each family's structure used
 *                    (scalar multiply, row scaling, rank-1 update), O(dk*dv)
 *                    per token.  Tests check that both agree.
 *
 *  All arithmetic is IEEE fp64.  Inputs are passed as fp64 arrays holding
 *  the exact values of whatever was stored (fp32 or bf16).
 *
 *  Layouts (row-major, last index fastest):
 *    k      [B][N][H][dk]        v    [B][N][H][dv]
 *    alpha  [B][N][H]  (scalar, dense)   or [B][N][H][dk]  (diagonal, KDA)
 *    beta   [B][N][H]  (dense, KDA; NULL means 1; ignored for scalar/diagonal)
 *    offsets[n_seg+1]  token offsets of the segments, offsets[0] = 0
 *    lam    [n_seg][B][H]     (scalar, dense, KDA)  or [n_seg][B][H][dk] (diag)
 *    That   [n_seg][B][H][dk][dk]   (dense and KDA)
 *    T      [n_seg][B][H][dk][dk]   plain T_C, all forms (optional)
 *    S      [n_seg][B][H][dk][dv]
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_SCALAR 0
#define ORACLE_DIAG 1
#define ORACLE_DENSE 2
#define ORACLE_KDA 3

/* largest gate of a token (the KDA form's per-token scale) */
static double max_gate(const double *at, int dk) {
  double m = at[0];
  for (int i = 1; i < dk; ++i)
    if (at[i] > m) m = at[i];
  return m;
}

/* ------------------------------------------------------------------ */
/* a tiny thread pool: run fn(ctx, i) for i in [0, n)                  */
/* ------------------------------------------------------------------ */
typedef void (*item_fn)(void *ctx, int64_t i);
typedef struct {
  item_fn fn;
  void *ctx;
  int64_t n;
  int64_t next;
  pthread_mutex_t mu;
} pool_t;

static void *pool_worker(void *arg) {
  pool_t *p = (pool_t *)arg;
  for (;;) {
    pthread_mutex_lock(&p->mu);
    int64_t i = p->next++;
    pthread_mutex_unlock(&p->mu);
    if (i >= p->n) return NULL;
    p->fn(p->ctx, i);
  }
}

static void run_items(item_fn fn, void *ctx, int64_t n, int n_threads) {
  if (n_threads < 1) n_threads = 1;
  if (n_threads > 256) n_threads = 256;
  if (n_threads > n) n_threads = (int)(n > 0 ? n : 1);
  pool_t p;
  p.fn = fn;
  p.ctx = ctx;
  p.n = n;
  p.next = 0;
  pthread_mutex_init(&p.mu, NULL);
  if (n_threads == 1) {
    pool_worker(&p);
  } else {
    pthread_t th[256];
    for (int t = 0; t < n_threads; ++t) pthread_create(&th[t], NULL, pool_worker, &p);
    for (int t = 0; t < n_threads; ++t) pthread_join(th[t], NULL);
  }
  pthread_mutex_destroy(&p.mu);
}

/* ------------------------------------------------------------------ */
/* per-token transition, literal form                                  */
/* ------------------------------------------------------------------ */

/* Fill Tt (dk x dk) with the token transition T_t of the given family,
 * and Th (dk x dk, may be NULL) with its ungated factor:
 *   scalar: T_t = a*I,            ungated I
 *   diag:   T_t = Diag(a[0..dk)), ungated I
 *   dense:  T_t = a*(I - b k k^T), ungated I - b k k^T
 *   KDA:    T_t = (I - b k k^T) Diag(a[0..dk)), ungated factor the same
 *           with a divided by its largest entry m_t (lambda adds ln m_t) */
static void token_transition(int form, int dk, const double *kt, const double *at, double bt,
                             double *Tt, double *Th) {
  for (int i = 0; i < dk; ++i) {
    for (int j = 0; j < dk; ++j) {
      double eye = (i == j) ? 1.0 : 0.0;
      double t, h;
      if (form == ORACLE_SCALAR) {
        t = at[0] * eye;
        h = eye;
      } else if (form == ORACLE_DIAG) {
        t = at[i] * eye;
        h = eye;
      } else if (form == ORACLE_KDA) {
        const double e = eye - bt * kt[i] * kt[j];
        t = e * at[j];
        h = e * (at[j] / max_gate(at, dk));
      } else {
        h = eye - bt * kt[i] * kt[j];
        t = at[0] * h;
      }
      Tt[i * dk + j] = t;
      if (Th) Th[i * dk + j] = h;
    }
  }
}

/* C = A(m x n) * B(n x p), all row-major, C must not alias. */
static void matmul(int m, int n, int p, const double *A, const double *B, double *C) {
  for (int i = 0; i < m; ++i) {
    for (int j = 0; j < p; ++j) {
      double acc = 0.0;
      for (int l = 0; l < n; ++l) acc += A[i * n + l] * B[l * p + j];
      C[i * p + j] = acc;
    }
  }
}

/* ------------------------------------------------------------------ */
/* build                                                               */
/* ------------------------------------------------------------------ */
typedef struct {
  int form, literal, B, H, dk, dv;
  int64_t N;
  const double *k, *v, *alpha, *beta;
  const int64_t *offsets;
  int n_seg;
  double *lam, *That, *T, *S;
  const double *q; /* prefill only: queries [B][N][H][dk] */
  double *O;       /* prefill only: outputs [B][N][H][dv], o_t = S_t^T q_t */
} build_ctx;

static inline const double *k_at(const build_ctx *c, int b, int64_t t, int h) {
  return c->k + (((int64_t)b * c->N + t) * c->H + h) * c->dk;
}
static inline const double *v_at(const build_ctx *c, int b, int64_t t, int h) {
  return c->v + (((int64_t)b * c->N + t) * c->H + h) * c->dv;
}
static inline const double *a_at(const build_ctx *c, int b, int64_t t, int h) {
  int64_t per = (c->form == ORACLE_DIAG || c->form == ORACLE_KDA) ? c->dk : 1;
  return c->alpha + (((int64_t)b * c->N + t) * c->H + h) * per;
}
static inline double b_at(const build_ctx *c, int b, int64_t t, int h) {
  if ((c->form != ORACLE_DENSE && c->form != ORACLE_KDA) || c->beta == NULL) return 1.0;
  return c->beta[((int64_t)b * c->N + t) * c->H + h];
}

/* One (segment, layer, head) unit.  Item index = (seg * B + b) * H + h,
 * which is also the unit's index in every output array. */
static void build_unit(void *vctx, int64_t item) {
  const build_ctx *c = (const build_ctx *)vctx;
  const int dk = c->dk, dv = c->dv, form = c->form;
  const int h = (int)(item % c->H);
  const int b = (int)((item / c->H) % c->B);
  const int seg = (int)(item / ((int64_t)c->H * c->B));
  const int64_t t0 = c->offsets[seg], t1 = c->offsets[seg + 1];
  const int nlam = (form == ORACLE_DIAG) ? dk : 1;

  double *S = (double *)calloc((size_t)dk * dv, sizeof(double));
  double *T = (double *)calloc((size_t)dk * dk, sizeof(double));  /* plain T_C */
  double *Th = (double *)calloc((size_t)dk * dk, sizeof(double)); /* ungated   */
  double *lam = (double *)calloc((size_t)nlam, sizeof(double));
  double *Tt = NULL, *Tht = NULL, *tmpS = NULL, *tmpT = NULL, *kS = NULL;
  if (c->literal) {
    Tt = (double *)malloc(sizeof(double) * dk * dk);
    Tht = (double *)malloc(sizeof(double) * dk * dk);
    tmpS = (double *)malloc(sizeof(double) * dk * (dk > dv ? dk : dv));
    tmpT = (double *)malloc(sizeof(double) * dk * dk);
  } else {
    kS = (double *)malloc(sizeof(double) * (dk > dv ? dk : dv));
  }
  /* T <- I, That <- I, S <- 0, lambda <- 0 */
  for (int i = 0; i < dk; ++i) {
    T[i * dk + i] = 1.0;
    Th[i * dk + i] = 1.0;
  }

  for (int64_t t = t0; t < t1; ++t) {
    const double *kt = k_at(c, b, t, h), *vt = v_at(c, b, t, h), *at = a_at(c, b, t, h);
    const double bt = b_at(c, b, t, h);
    if (form == ORACLE_KDA)
      lam[0] += log(max_gate(at, dk));
    else
      for (int i = 0; i < nlam; ++i) lam[i] += log(at[i]);
    if (c->literal) {
      /* S <- T_t S + bt * k v^T ; T <- T_t T ; That <- That_t That */
      token_transition(form, dk, kt, at, bt, Tt, Tht);
      matmul(dk, dk, dv, Tt, S, tmpS);
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) S[i * dv + j] = tmpS[i * dv + j] + bt * kt[i] * vt[j];
      matmul(dk, dk, dk, Tt, T, tmpT);
      memcpy(T, tmpT, sizeof(double) * dk * dk);
      matmul(dk, dk, dk, Tht, Th, tmpT);
      memcpy(Th, tmpT, sizeof(double) * dk * dk);
    } else if (form == ORACLE_SCALAR) {
      /* T_t = a I : every entry of S and T scales by a */
      const double a = at[0];
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) S[i * dv + j] = a * S[i * dv + j] + kt[i] * vt[j];
      for (int i = 0; i < dk * dk; ++i) T[i] *= a;
    } else if (form == ORACLE_DIAG) {
      /* T_t = Diag(a) : row i of S and of T scales by a[i] */
      for (int i = 0; i < dk; ++i) {
        for (int j = 0; j < dv; ++j) S[i * dv + j] = at[i] * S[i * dv + j] + kt[i] * vt[j];
        for (int j = 0; j < dk; ++j) T[i * dk + j] *= at[i];
      }
    } else if (form == ORACLE_KDA) {
      /* T_t = (I - b k k^T) Diag(a): scale the rows of S and T by a and
       * those of That by a / m, then X <- X - b k (k^T X) for all three;
       * then S += b k v^T */
      const double m = max_gate(at, dk);
      for (int i = 0; i < dk; ++i) {
        for (int j = 0; j < dv; ++j) S[i * dv + j] *= at[i];
        for (int j = 0; j < dk; ++j) {
          T[i * dk + j] *= at[i];
          Th[i * dk + j] *= at[i] / m;
        }
      }
      double *X[3] = {S, T, Th};
      const int W[3] = {dv, dk, dk};
      for (int x = 0; x < 3; ++x) {
        for (int j = 0; j < W[x]; ++j) {
          double s = 0.0;
          for (int i = 0; i < dk; ++i) s += kt[i] * X[x][i * W[x] + j];
          kS[j] = s;
        }
        for (int i = 0; i < dk; ++i)
          for (int j = 0; j < W[x]; ++j) X[x][i * W[x] + j] -= bt * kt[i] * kS[j];
      }
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) S[i * dv + j] += bt * kt[i] * vt[j];
    } else {
      /* T_t = a (I - b k k^T):  X <- a (X - b k (k^T X)) for X = S, T;
       * That <- That - b k (k^T That);  then S += b k v^T */
      const double a = at[0];
      for (int j = 0; j < dv; ++j) {
        double s = 0.0;
        for (int i = 0; i < dk; ++i) s += kt[i] * S[i * dv + j];
        kS[j] = s;
      }
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
          S[i * dv + j] = a * (S[i * dv + j] - bt * kt[i] * kS[j]) + bt * kt[i] * vt[j];
      for (int j = 0; j < dk; ++j) {
        double s = 0.0;
        for (int i = 0; i < dk; ++i) s += kt[i] * T[i * dk + j];
        kS[j] = s;
      }
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dk; ++j) T[i * dk + j] = a * (T[i * dk + j] - bt * kt[i] * kS[j]);
      for (int j = 0; j < dk; ++j) {
        double s = 0.0;
        for (int i = 0; i < dk; ++i) s += kt[i] * Th[i * dk + j];
        kS[j] = s;
      }
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dk; ++j) Th[i * dk + j] -= bt * kt[i] * kS[j];
    }
    if (c->O) {
      /* the token's output reads the state after its own update:
       * o_t = S_t^T q_t */
      const double *qt = c->q + (((int64_t)b * c->N + t) * c->H + h) * dk;
      double *ot = c->O + (((int64_t)b * c->N + t) * c->H + h) * dv;
      for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i) acc += qt[i] * S[i * dv + j];
        ot[j] = acc;
      }
    }
  }

  memcpy(c->S + item * dk * dv, S, sizeof(double) * dk * dv);
  memcpy(c->lam + item * nlam, lam, sizeof(double) * nlam);
  if (c->That) memcpy(c->That + item * dk * dk, Th, sizeof(double) * dk * dk);
  if (c->T) memcpy(c->T + item * dk * dk, T, sizeof(double) * dk * dk);
  free(S);
  free(T);
  free(Th);
  free(lam);
  free(Tt);
  free(Tht);
  free(tmpS);
  free(tmpT);
  free(kS);
}

/* Build the pair of every (segment, layer, head).  Returns 0, or -1 on bad
 * arguments.  That may be NULL (it is only meaningful for the dense form;
 * for scalar/diag the ungated factor is I), T may be NULL. */
int oracle_build(int form, int literal, int B, int H, int dk, int dv, int64_t N, const double *k,
                 const double *v, const double *alpha, const double *beta, const int64_t *offsets,
                 int n_seg, double *lam, double *That, double *T, double *S, int n_threads) {
  if (form < 0 || form > 3 || B < 0 || H < 0 || dk <= 0 || dv <= 0 || n_seg < 0) return -1;
  if (offsets[0] != 0 || offsets[n_seg] != N) return -1;
  for (int i = 0; i < n_seg; ++i)
    if (offsets[i + 1] < offsets[i]) return -1;
  build_ctx c = {form, literal, B, H, dk, dv, N, k, v, alpha, beta, offsets, n_seg, lam, That, T, S};
  run_items(build_unit, &c, (int64_t)n_seg * B * H, n_threads);
  return 0;
}

/* Independent prefill of every segment with outputs: the build above, and
 * for every token the output of the state right after its own update,
 * o_t = S_t^T q_t, with the state starting from zero at each segment's first
 * token (a cached segment is prefilled on its own).  O [B][N][H][dv]. */
int oracle_prefill(int form, int literal, int B, int H, int dk, int dv, int64_t N,
                   const double *q, const double *k, const double *v, const double *alpha,
                   const double *beta, const int64_t *offsets, int n_seg, double *lam,
                   double *That, double *T, double *S, double *O, int n_threads) {
  if (form < 0 || form > 3 || B < 0 || H < 0 || dk <= 0 || dv <= 0 || n_seg < 0) return -1;
  if (!q || !O) return -1;
  if (offsets[0] != 0 || offsets[n_seg] != N) return -1;
  for (int i = 0; i < n_seg; ++i)
    if (offsets[i + 1] < offsets[i]) return -1;
  build_ctx c = {form, literal, B, H, dk, dv, N, k, v, alpha, beta, offsets, n_seg, lam, That, T, S};
  c.q = q;
  c.O = O;
  run_items(build_unit, &c, (int64_t)n_seg * B * H, n_threads);
  return 0;
}

/* ------------------------------------------------------------------ */
/* unsplit recurrence: the state after all N tokens from S_in          */
/* ------------------------------------------------------------------ */
typedef struct {
  build_ctx bc;
  const double *S_in; /* [B][H][dk][dv] or NULL */
  double *S_out;      /* [B][H][dk][dv] */
} rec_ctx;

static void recurrence_unit(void *vctx, int64_t item) {
  const rec_ctx *r = (const rec_ctx *)vctx;
  const build_ctx *c = &r->bc;
  const int dk = c->dk, dv = c->dv, form = c->form;
  const int h = (int)(item % c->H), b = (int)(item / c->H);
  double *S = r->S_out + item * dk * dv;
  if (r->S_in)
    memcpy(S, r->S_in + item * dk * dv, sizeof(double) * dk * dv);
  else
    memset(S, 0, sizeof(double) * dk * dv);
  double *Tt = (double *)malloc(sizeof(double) * dk * dk);
  double *tmp = (double *)malloc(sizeof(double) * dk * dv);
  for (int64_t t = 0; t < c->N; ++t) {
    const double *kt = k_at(c, b, t, h), *vt = v_at(c, b, t, h), *at = a_at(c, b, t, h);
    const double bt = b_at(c, b, t, h);
    token_transition(form, dk, kt, at, bt, Tt, NULL);
    matmul(dk, dk, dv, Tt, S, tmp);
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) S[i * dv + j] = tmp[i * dv + j] + bt * kt[i] * vt[j];
  }
  free(Tt);
  free(tmp);
}

/* Literal per-token recurrence over all N tokens of every (layer, head),
 * started from S_in (NULL = zero). */
int oracle_recurrence(int form, int B, int H, int dk, int dv, int64_t N, const double *k,
                      const double *v, const double *alpha, const double *beta,
                      const double *S_in, double *S_out, int n_threads) {
  if (form < 0 || form > 3 || dk <= 0 || dv <= 0) return -1;
  rec_ctx r;
  memset(&r, 0, sizeof(r));
  r.bc.form = form;
  r.bc.B = B;
  r.bc.H = H;
  r.bc.dk = dk;
  r.bc.dv = dv;
  r.bc.N = N;
  r.bc.k = k;
  r.bc.v = v;
  r.bc.alpha = alpha;
  r.bc.beta = beta;
  r.S_in = S_in;
  r.S_out = S_out;
  run_items(recurrence_unit, &r, (int64_t)B * H, n_threads);
  return 0;
}

/* ------------------------------------------------------------------ */
/* compose and naive add over chains of cached pairs                   */
/* ------------------------------------------------------------------ */
/* Pool layouts: lam [P][B][H] (diag: [P][B][H][dk]); That [P][B][H][dk][dk]
 * (dense only); S [P][B][H][dk][dv].  Chains: request r uses pool entries
 * idx[chain_off[r] .. chain_off[r+1]) in that order (first applied first).
 * S_in/S_out: [R][B][H][dk][dv]; S_in NULL = zero. */
typedef struct {
  int form, B, H, dk, dv, naive;
  const double *lam, *That, *S;
  const int64_t *off;
  const int32_t *idx;
  const double *S_in;
  double *S_out, *lam_out, *That_out;
} comp_ctx;

static void compose_unit(void *vctx, int64_t item) {
  const comp_ctx *c = (const comp_ctx *)vctx;
  const int dk = c->dk, dv = c->dv, form = c->form;
  const int64_t BH = (int64_t)c->B * c->H;
  const int64_t r = item / BH, bh = item % BH;
  const int nlam = (form == ORACLE_DIAG) ? dk : 1;
  double *S = c->S_out + item * dk * dv;
  if (c->S_in)
    memcpy(S, c->S_in + item * dk * dv, sizeof(double) * dk * dv);
  else
    memset(S, 0, sizeof(double) * dk * dv);
  double *tmp = (double *)malloc(sizeof(double) * dk * dv);
  double *T = (double *)malloc(sizeof(double) * dk * dk);
  double *Tacc = (double *)calloc((size_t)dk * dk, sizeof(double));
  double *Ttmp = (double *)malloc(sizeof(double) * dk * dk);
  double *lacc = (double *)calloc((size_t)nlam, sizeof(double));
  for (int i = 0; i < dk; ++i) Tacc[i * dk + i] = 1.0;

  for (int64_t s = c->off[r]; s < c->off[r + 1]; ++s) {
    const int64_t p = c->idx[s];
    const int64_t unit = p * BH + bh;
    const double *Sp = c->S + unit * dk * dv;
    if (c->naive) {
      /* naive ablation: S <- S + S(C|0) */
      for (int i = 0; i < dk * dv; ++i) S[i] += Sp[i];
      continue;
    }
    const double *lp = c->lam + unit * nlam;
    /* the pair's operator T_C = e^lambda * That (That = I for scalar/diag) */
    for (int i = 0; i < dk; ++i) {
      for (int j = 0; j < dk; ++j) {
        double eye = (i == j) ? 1.0 : 0.0;
        double th = (form == ORACLE_DENSE || form == ORACLE_KDA) ? c->That[unit * dk * dk + i * dk + j] : eye;
        double scale = exp(lp[form == ORACLE_DIAG ? i : 0]);
        T[i * dk + j] = scale * th;
      }
    }
    /* S <- T_C S + S(C|0) */
    matmul(dk, dk, dv, T, S, tmp);
    for (int i = 0; i < dk * dv; ++i) S[i] = tmp[i] + Sp[i];
    /* the chain's own pair: lambda sums, That multiplies on the left */
    for (int i = 0; i < nlam; ++i) lacc[i] += lp[i];
    if (form == ORACLE_DENSE || form == ORACLE_KDA) {
      matmul(dk, dk, dk, c->That + unit * dk * dk, Tacc, Ttmp);
      memcpy(Tacc, Ttmp, sizeof(double) * dk * dk);
    }
  }
  if (c->lam_out) memcpy(c->lam_out + item * nlam, lacc, sizeof(double) * nlam);
  if (c->That_out) memcpy(c->That_out + item * dk * dk, Tacc, sizeof(double) * dk * dk);
  free(tmp);
  free(T);
  free(Tacc);
  free(Ttmp);
  free(lacc);
}

static int check_chains(int64_t P, int n_req, const int64_t *off, const int32_t *idx) {
  if (n_req < 0 || off[0] != 0) return -1;
  for (int r = 0; r < n_req; ++r) {
    if (off[r + 1] < off[r]) return -1;
    for (int64_t s = off[r]; s < off[r + 1]; ++s)
      if (idx[s] < 0 || idx[s] >= P) return -1;
  }
  return 0;
}

/* S_out[r] = T_{p_n} ( ... (T_{p_1} S_in[r] + S_{p_1}) ... ) + S_{p_n}.
 * lam_out / That_out (nullable) receive the chain's own pair. */
int oracle_compose(int form, int B, int H, int dk, int dv, int64_t P, const double *lam,
                   const double *That, const double *S, int n_req, const int64_t *chain_off,
                   const int32_t *chain_idx, const double *S_in, double *S_out, double *lam_out,
                   double *That_out, int n_threads) {
  if (form < 0 || form > 3 || check_chains(P, n_req, chain_off, chain_idx)) return -1;
  if ((form == ORACLE_DENSE || form == ORACLE_KDA) && That == NULL) return -1;
  comp_ctx c = {form, B,         H,       dk,   dv,    0,       lam,    That,
                S,    chain_off, chain_idx, S_in, S_out, lam_out, That_out};
  run_items(compose_unit, &c, (int64_t)n_req * B * H, n_threads);
  return 0;
}

/* S_out[r] = S_in[r] + sum over the chain of S(C|0). */
int oracle_naive_add(int B, int H, int dk, int dv, int64_t P, const double *S, int n_req,
                     const int64_t *chain_off, const int32_t *chain_idx, const double *S_in,
                     double *S_out, int n_threads) {
  if (check_chains(P, n_req, chain_off, chain_idx)) return -1;
  comp_ctx c = {ORACLE_SCALAR, B,         H,         dk,   dv,    1,    NULL, NULL,
                S,             chain_off, chain_idx, S_in, S_out, NULL, NULL};
  run_items(compose_unit, &c, (int64_t)n_req * B * H, n_threads);
  return 0;
}

/* ------------------------------------------------------------------ */
/* reuse with seam windows                                             */
/* ------------------------------------------------------------------ */
/* On reuse, the first few tokens of a cached segment (its seam window) are
 * not part of the cached pair: they are run again from the running state,
 * token by token, and each of them emits its layer output; then the pair of
 * the rest of the segment is applied.
 *   [xix.ai HYPIC article (French), paragraph on full-attention layers: a
 *    window of w tokens (8 by default) at the start of every inner segment is
 *    left out of the cache and recomputed under the full prefix on reuse;
 *    the linear layers advance the running state through these tokens and
 *    pass each token's per-layer output up to the attention layer above.]
 * The output of a token is read from the state after its own update (the
 * usual linear-attention readout):  o_t = S_t^T q_t,  o_t in R^{dv}.
 *
 * Chain entry c of request r: first its seam tokens
 * [seam_off[c], seam_off[c+1]) of the seam arrays, then pool pair idx[c].
 * Seam inputs use the build layout with N = NS (the seam token count):
 * q, k [B][NS][H][dk], v [B][NS][H][dv], alpha, beta as in the build.
 * O [B][NS][H][dv].  literal = 1 applies each seam token as an explicit
 * transition matrix; 0 uses the family's structure (as in the build). */
typedef struct {
  comp_ctx cc;
  build_ctx tok; /* the seam inputs (offsets unused) */
  int literal;
  const int64_t *seam_off;
  const double *q;
  double *O;
} seam_ctx;

static void seam_token(const seam_ctx *sc, int b, int h, int64_t t, double *S, double *Tt,
                       double *tmp) {
  const build_ctx *c = &sc->tok;
  const int dk = c->dk, dv = c->dv, form = c->form;
  const double *kt = k_at(c, b, t, h), *vt = v_at(c, b, t, h), *at = a_at(c, b, t, h);
  const double bt = b_at(c, b, t, h);
  if (sc->literal) {
    token_transition(form, dk, kt, at, bt, Tt, NULL);
    matmul(dk, dk, dv, Tt, S, tmp);
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) S[i * dv + j] = tmp[i * dv + j] + bt * kt[i] * vt[j];
  } else if (form == ORACLE_KDA) {
    /* S <- (I - b k k^T) Diag(a) S + b k v^T: the rows scaled by their gates,
       then the erase along k and the write */
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) S[i * dv + j] *= at[i];
    for (int j = 0; j < dv; ++j) {
      double s = 0.0;
      for (int i = 0; i < dk; ++i) s += kt[i] * S[i * dv + j];
      tmp[j] = s;
    }
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j) S[i * dv + j] += bt * kt[i] * (vt[j] - tmp[j]);
  } else if (form == ORACLE_DENSE) {
    /* S <- a (S - b k (k^T S)) + b k v^T */
    for (int j = 0; j < dv; ++j) {
      double s = 0.0;
      for (int i = 0; i < dk; ++i) s += kt[i] * S[i * dv + j];
      tmp[j] = s;
    }
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dv; ++j)
        S[i * dv + j] = at[0] * (S[i * dv + j] - bt * kt[i] * tmp[j]) + bt * kt[i] * vt[j];
  } else {
    /* scalar: every row decays by a[0]; diagonal: row i by a[i] */
    for (int i = 0; i < dk; ++i) {
      const double ai = (form == ORACLE_DIAG) ? at[i] : at[0];
      for (int j = 0; j < dv; ++j) S[i * dv + j] = ai * S[i * dv + j] + kt[i] * vt[j];
    }
  }
  /* o_t = S_t^T q_t */
  const double *qt = sc->q + (((int64_t)b * c->N + t) * c->H + h) * dk;
  double *ot = sc->O + (((int64_t)b * c->N + t) * c->H + h) * dv;
  for (int j = 0; j < dv; ++j) {
    double s = 0.0;
    for (int i = 0; i < dk; ++i) s += qt[i] * S[i * dv + j];
    ot[j] = s;
  }
}

static void seam_unit(void *vctx, int64_t item) {
  const seam_ctx *sc = (const seam_ctx *)vctx;
  const comp_ctx *c = &sc->cc;
  const int dk = c->dk, dv = c->dv, form = c->form;
  const int64_t BH = (int64_t)c->B * c->H;
  const int64_t r = item / BH, bh = item % BH;
  const int b = (int)(bh / c->H), h = (int)(bh % c->H);
  double *S = c->S_out + item * dk * dv;
  if (c->S_in)
    memcpy(S, c->S_in + item * dk * dv, sizeof(double) * dk * dv);
  else
    memset(S, 0, sizeof(double) * dk * dv);
  const int dmax = dk > dv ? dk : dv;
  double *Tt = (double *)malloc(sizeof(double) * dk * dk);
  double *tmp = (double *)malloc(sizeof(double) * dk * dmax);
  double *Tp = (double *)malloc(sizeof(double) * dk * dk);
  for (int64_t e = c->off[r]; e < c->off[r + 1]; ++e) {
    for (int64_t t = sc->seam_off[e]; t < sc->seam_off[e + 1]; ++t)
      seam_token(sc, b, h, t, S, Tt, tmp);
    /* then the cached pair of the rest of the segment: S <- T_p S + S_p */
    const int64_t unit = (int64_t)c->idx[e] * BH + bh;
    const int nlam = (form == ORACLE_DIAG) ? dk : 1;
    const double *lp = c->lam + unit * nlam;
    for (int i = 0; i < dk; ++i)
      for (int j = 0; j < dk; ++j) {
        const double ungated = (form == ORACLE_DENSE || form == ORACLE_KDA)
                                   ? c->That[unit * dk * dk + i * dk + j]
                                   : (double)(i == j);
        Tp[i * dk + j] = exp(lp[nlam == 1 ? 0 : i]) * ungated;
      }
    matmul(dk, dk, dv, Tp, S, tmp);
    const double *Sp = c->S + unit * dk * dv;
    for (int i = 0; i < dk * dv; ++i) S[i] = tmp[i] + Sp[i];
  }
  free(Tt);
  free(tmp);
  free(Tp);
}

int oracle_seam_compose(int form, int literal, int B, int H, int dk, int dv, int64_t P,
                        const double *lam, const double *That, const double *S, int n_req,
                        const int64_t *chain_off, const int32_t *chain_idx,
                        const int64_t *seam_off, int64_t NS, const double *q, const double *k,
                        const double *v, const double *alpha, const double *beta,
                        const double *S_in, double *S_out, double *O, int n_threads) {
  if (form < 0 || form > 3 || dk <= 0 || dv <= 0 || check_chains(P, n_req, chain_off, chain_idx))
    return -1;
  if ((form == ORACLE_DENSE || form == ORACLE_KDA) && That == NULL) return -1;
  const int64_t total = chain_off[n_req];
  if (seam_off[0] != 0 || seam_off[total] != NS) return -1;
  for (int64_t e = 0; e < total; ++e)
    if (seam_off[e + 1] < seam_off[e]) return -1;
  seam_ctx sc;
  memset(&sc, 0, sizeof(sc));
  comp_ctx cc = {form,      B,         H,    dk,    dv,   0,    lam, That,
                 S,         chain_off, chain_idx, S_in, S_out, NULL, NULL};
  sc.cc = cc;
  sc.tok.form = form;
  sc.tok.B = B;
  sc.tok.H = H;
  sc.tok.dk = dk;
  sc.tok.dv = dv;
  sc.tok.N = NS;
  sc.tok.k = k;
  sc.tok.v = v;
  sc.tok.alpha = alpha;
  sc.tok.beta = beta;
  sc.literal = literal;
  sc.seam_off = seam_off;
  sc.q = q;
  sc.O = O;
  run_items(seam_unit, &sc, (int64_t)n_req * B * H, n_threads);
  return 0;
}
