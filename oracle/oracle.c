/*
 * Oracle for the lightning-indexer hot path: plain, slow, fp64, on the CPU.
 *
 * TEST INFRASTRUCTURE ONLY.  Tests, the smoke check and the benchmark's CPU
 * baseline call this; the product library never does, and this file shares no
 * source, header or table with it.
 *
 * Sources (web pages; cited by title and section):
 *   [LC]  "Long context", llm-serving.xyz lecture 03, section "The Architectural
 *         Answer: Read Less of the Past": paragraph "Stage 1, the lightning
 *         indexer" (one 128-d FP8 key per token shared by 64 heads, 132 B per
 *         token, weighted-ReLU score of every past key, output is a ranking) and
 *         paragraph "Stage 2, sparse main attention" (exact attention over the
 *         top-k keys only); Derivation 4 (bytes and FLOPs per key); section
 *         "Sparsity Is a Systems Feature: The Blast Radius", "Kernel layer"
 *         (indexer scoring -> fused top-k -> sparse attention gather by index).
 *   [LS]  LeanSparse podcast transcript, cues 01:33-02:06 (top-k before attention,
 *         k = 512) and 07:12-08:00 (compact keys, a 2,048-candidate coarse pass,
 *         then an exact rerank of the original keys down to 512).
 *   [LSA] "Latent Sparse Attention" article, section "What the kernels do about
 *         the top-p": selection over packed keys with the score above an inverted
 *         id, so equal scores prefer the smaller id.
 *
 * Readings where the pages are silent (each one is listed in the design notes):
 *   - fp8 is OCP E4M3FN (bias 7, max 448, no infinities); a stored key is
 *     code * row scale, exact in fp64.
 *   - every sum is an fma chain in ascending index order, starting from 0:
 *     dot_h = chain_j(q[h][j], k[j]); score = chain_h(w[h], max(dot_h, 0)).
 *   - the top-k set is the first k entries in the order (score descending, index
 *     ascending), i.e. equal scores prefer the smaller index; it is returned in
 *     ascending index order (attention does not depend on the order); rows with
 *     fewer than k visible keys are padded with (-1, -inf); invisible keys score
 *     -inf.
 *   - compact stage 1 scores the weighted-ReLU form in the projected space with
 *     int8 query codes: y_h = P q_h (fma chain over j), qs_h = max|y_h| / 127
 *     (1 if zero), q8_h = rint(y_h / qs_h), W_h = w_h * qs_h, D = q8_h . c_s
 *     (exact int), s1 = cs_s * chain_h(W_h, max(D_h, 0)); stage 2 rescores the
 *     shortlist with the exact score above.
 *   - sparse attention: l_i = tau * q . kv_i over all dqk elements, values are the
 *     first dv elements of the same row, entries with index -1 are skipped.
 *
 * Parity pins live in the CPU tests (hand-computed scores, exact rationals, closed
 * forms, invariants).  Recall values of the compact search are parity unpinned:
 * the pages print none for this encoding.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_FP8_E4M3 = 2, ORC_I8 = 3 };

/* ---- decoders (from the format definitions) -------------------------------- */

double orc_dec_bf16(uint16_t b) {
  /* bf16 is the upper half of an IEEE binary32 */
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

double orc_dec_e4m3(uint8_t c) {
  /* OCP 8-bit floating point, E4M3 "FN": 1 sign, 4 exponent (bias 7), 3
   * mantissa bits; exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN;
   * there are no infinities. */
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp((double)m, -9);
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

static double load_elem(const void *p, int type, int64_t i) {
  switch (type) {
    case ORC_F32: return (double)((const float *)p)[i];
    case ORC_BF16: return orc_dec_bf16(((const uint16_t *)p)[i]);
    case ORC_FP8_E4M3: return orc_dec_e4m3(((const uint8_t *)p)[i]);
    case ORC_I8: return (double)((const int8_t *)p)[i];
  }
  return NAN;
}

/* ---- threads over rows ---------------------------------------------------------- */

static int g_threads_used = 1;

static int n_threads(void) {
  const char *s = getenv("ORACLE_THREADS");
  long n = s ? atol(s) : sysconf(_SC_NPROCESSORS_ONLN);
  if (n < 1) n = 1;
  if (n > 16) n = 16;
  return (int)n;
}

int orc_threads_used(void) { return g_threads_used; }

typedef void (*row_fn)(void *ctx, int64_t row);
typedef struct { row_fn fn; void *ctx; int64_t next, n; pthread_mutex_t mu; } pool_t;

static void *pool_worker(void *p) {
  pool_t *pl = (pool_t *)p;
  for (;;) {
    pthread_mutex_lock(&pl->mu);
    int64_t r = pl->next++;
    pthread_mutex_unlock(&pl->mu);
    if (r >= pl->n) break;
    pl->fn(pl->ctx, r);
  }
  return NULL;
}

/* Rows are independent; each row is computed wholly by one thread, so results do
 * not depend on the thread count. */
static void for_rows(int64_t n, row_fn fn, void *ctx) {
  int nt = n_threads();
  if (n < nt) nt = (int)(n > 0 ? n : 1);
  g_threads_used = nt;
  pool_t pl = {fn, ctx, 0, n};
  pthread_mutex_init(&pl.mu, NULL);
  if (nt == 1) {
    pool_worker(&pl);
  } else {
    pthread_t th[16];
    for (int t = 0; t < nt; ++t) pthread_create(&th[t], NULL, pool_worker, &pl);
    for (int t = 0; t < nt; ++t) pthread_join(th[t], NULL);
  }
  pthread_mutex_destroy(&pl.mu);
}

/* ---- O1: lightning-indexer score [LC "Stage 1, the lightning indexer"] ---------- */

/* score(q, w, key) = sum_h w[h] * max(q[h] . key, 0), every sum an ascending fma
 * chain.  qd: [H, d] queries, key: [d], both already decoded to fp64. */
static double score_one(const double *qd, const double *wd, const double *key, int64_t H, int64_t d) {
  double acc = 0.0;
  for (int64_t h = 0; h < H; ++h) {
    double dot = 0.0;
    for (int64_t j = 0; j < d; ++j) dot = fma(qd[h * d + j], key[j], dot);
    acc = fma(wd[h], dot > 0.0 ? dot : 0.0, acc);
  }
  return acc;
}

typedef struct {
  const void *q; int q_type; const float *w;
  const void *k; int k_type; const float *k_scale; const int32_t *nv;
  int64_t B, T, S, H, d;
  double *scores;
} score_ctx;

static void score_row(void *p, int64_t r) {
  score_ctx *c = (score_ctx *)p;
  int64_t b = r / c->T, H = c->H, d = c->d, S = c->S;
  double *qd = (double *)malloc(sizeof(double) * H * d);
  double *wd = (double *)malloc(sizeof(double) * H);
  double *key = (double *)malloc(sizeof(double) * d);
  for (int64_t i = 0; i < H * d; ++i) qd[i] = load_elem(c->q, c->q_type, r * H * d + i);
  for (int64_t h = 0; h < H; ++h) wd[h] = (double)c->w[r * H + h];
  int64_t nv = c->nv ? c->nv[r] : S;
  if (nv > S) nv = S;
  for (int64_t s = 0; s < S; ++s) {
    if (s >= nv) { c->scores[r * S + s] = -INFINITY; continue; }
    int64_t row = b * S + s;
    double sc = c->k_scale ? (double)c->k_scale[row] : 1.0;
    for (int64_t j = 0; j < d; ++j) key[j] = load_elem(c->k, c->k_type, row * d + j) * sc;
    c->scores[r * S + s] = score_one(qd, wd, key, H, d);
  }
  free(qd); free(wd); free(key);
}

/* q: [B, T, H, d] (q_type), w: [B, T, H] fp32, k: [B, S, d] (k_type),
 * k_scale: [B, S] fp32 or NULL (= 1), nv: [B*T] visible-key counts or NULL (= S).
 * scores: [B*T, S] fp64; keys s >= nv[row] get -inf. */
void orc_indexer_score(const void *q, int q_type, const float *w, const void *k, int k_type,
                       const float *k_scale, const int32_t *nv, int64_t B, int64_t T, int64_t S,
                       int64_t H, int64_t d, double *scores) {
  score_ctx c = {q, q_type, w, k, k_type, k_scale, nv, B, T, S, H, d, scores};
  for_rows(B * T, score_row, &c);
}

/* ---- O2: top-k [LC "Stage 2, sparse main attention"; LSA packed-key order] ------- */

typedef struct { double v; int32_t i; } pair_t;

static int cmp_index(const void *a, const void *b) {
  const pair_t *x = (const pair_t *)a, *y = (const pair_t *)b;
  return (x->i < y->i) ? -1 : (x->i > y->i);
}

static int cmp_desc(const void *a, const void *b) {
  const pair_t *x = (const pair_t *)a, *y = (const pair_t *)b;
  if (x->v > y->v) return -1;
  if (x->v < y->v) return 1;
  return (x->i < y->i) ? -1 : (x->i > y->i);
}

/* The min(k, n) best of the first n entries of one row by (score desc, index
 * asc), returned in ascending index order, padded with (-1, -inf). */
static void topk_one(const double *row, int64_t n, int64_t k, int32_t *idx, double *val) {
  pair_t *p = (pair_t *)malloc(sizeof(pair_t) * (n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) { p[i].v = row[i]; p[i].i = (int32_t)i; }
  qsort(p, (size_t)n, sizeof(pair_t), cmp_desc);
  qsort(p, (size_t)(n < k ? n : k), sizeof(pair_t), cmp_index);
  for (int64_t j = 0; j < k; ++j) {
    if (j < n) { idx[j] = p[j].i; if (val) val[j] = p[j].v; }
    else { idx[j] = -1; if (val) val[j] = -INFINITY; }
  }
  free(p);
}

typedef struct { const double *scores; const int32_t *nv; int64_t S, k; int32_t *idx; double *val; } topk_ctx;

static void topk_row(void *p, int64_t r) {
  topk_ctx *c = (topk_ctx *)p;
  int64_t n = c->nv ? c->nv[r] : c->S;
  if (n > c->S) n = c->S;
  if (n < 0) n = 0;
  topk_one(c->scores + r * c->S, n, c->k, c->idx + r * c->k, c->val ? c->val + r * c->k : NULL);
}

/* scores: [R, S]; nv: [R] or NULL; idx: [R, k]; val: [R, k] or NULL. */
void orc_topk(const double *scores, const int32_t *nv, int64_t R, int64_t S, int64_t k, int32_t *idx,
              double *val) {
  topk_ctx c = {scores, nv, S, k, idx, val};
  for_rows(R, topk_row, &c);
}

/* ---- O3: compact search + exact rerank [LS 07:12-08:00] ---------------------------- */

/* Query side of stage 1 for one (b, h): project, scale, round to int8. */
static void compact_query_one(const uint16_t *q, float w, const float *P, int64_t d, int64_t dc,
                              int8_t *q8, double *qs, double *W) {
  double y[256];
  double amax = 0.0;
  for (int64_t i = 0; i < dc; ++i) {
    double acc = 0.0;
    for (int64_t j = 0; j < d; ++j) acc = fma((double)P[i * d + j], orc_dec_bf16(q[j]), acc);
    y[i] = acc;
    if (fabs(acc) > amax) amax = fabs(acc);
  }
  double s = amax > 0.0 ? amax / 127.0 : 1.0;
  for (int64_t i = 0; i < dc; ++i) {
    double t = rint(y[i] / s);
    if (t > 127.0) t = 127.0;
    if (t < -127.0) t = -127.0;
    q8[i] = (int8_t)t;
  }
  *qs = s;
  *W = (double)w * s;
}

/* q: [B, H, d] bf16, w: [B, H], P: [dc, d] -> q8: [B, H, dc], qs, W: [B, H]. */
void orc_compact_query(const uint16_t *q, const float *w, const float *P, int64_t B, int64_t H, int64_t d,
                       int64_t dc, int8_t *q8, double *qs, double *W) {
  for (int64_t r = 0; r < B * H; ++r)
    compact_query_one(q + r * d, w[r], P, d, dc, q8 + r * dc, qs + r, W + r);
}

static double stage1_one(const int8_t *q8, const double *W, const int8_t *c, float cs, int64_t H, int64_t dc) {
  double acc = 0.0;
  for (int64_t h = 0; h < H; ++h) {
    int64_t D = 0;
    for (int64_t i = 0; i < dc; ++i) D += (int64_t)q8[h * dc + i] * (int64_t)c[i];
    acc = fma(W[h], (double)(D > 0 ? D : 0), acc);
  }
  return (double)cs * acc;
}

typedef struct {
  const uint16_t *q; const float *w; const float *P; const int8_t *c; const float *cs;
  const uint16_t *kf; const int32_t *nv; int64_t S, H, d, dc, m, k;
  int32_t *shortlist; int32_t *idx; double *val; double *s1_out;
} compact_ctx;

static void compact_row(void *p, int64_t b) {
  compact_ctx *c = (compact_ctx *)p;
  int64_t S = c->S, H = c->H, d = c->d, dc = c->dc, m = c->m, k = c->k;
  int8_t *q8 = (int8_t *)malloc((size_t)(H * dc));
  double *qs = (double *)malloc(sizeof(double) * H);
  double *W = (double *)malloc(sizeof(double) * H);
  for (int64_t h = 0; h < H; ++h)
    compact_query_one(c->q + (b * H + h) * d, c->w[b * H + h], c->P, d, dc, q8 + h * dc, qs + h, W + h);
  int64_t nv = c->nv ? c->nv[b] : S;
  if (nv > S) nv = S;
  /* stage 1: coarse score of every visible key, keep the top m */
  double *s1 = (double *)malloc(sizeof(double) * (nv > 0 ? nv : 1));
  for (int64_t s = 0; s < nv; ++s) s1[s] = stage1_one(q8, W, c->c + (b * S + s) * dc, c->cs[b * S + s], H, dc);
  if (c->s1_out)
    for (int64_t s = 0; s < S; ++s) c->s1_out[b * S + s] = s < nv ? s1[s] : -INFINITY;
  int32_t *sl = c->shortlist + b * m;
  topk_one(s1, nv, m, sl, NULL);
  /* stage 2: exact score of the shortlisted keys (original bf16 keys), keep top k */
  double *qd = (double *)malloc(sizeof(double) * H * d);
  double *wd = (double *)malloc(sizeof(double) * H);
  double *key = (double *)malloc(sizeof(double) * d);
  for (int64_t i = 0; i < H * d; ++i) qd[i] = orc_dec_bf16(c->q[b * H * d + i]);
  for (int64_t h = 0; h < H; ++h) wd[h] = (double)c->w[b * H + h];
  int64_t nm = nv < m ? nv : m;
  pair_t *pr = (pair_t *)malloc(sizeof(pair_t) * (nm > 0 ? nm : 1));
  for (int64_t i = 0; i < nm; ++i) {
    int64_t s = sl[i];
    for (int64_t j = 0; j < d; ++j) key[j] = orc_dec_bf16(c->kf[(b * S + s) * d + j]);
    pr[i].v = score_one(qd, wd, key, H, d);
    pr[i].i = (int32_t)s;
  }
  qsort(pr, (size_t)nm, sizeof(pair_t), cmp_desc);
  qsort(pr, (size_t)(nm < k ? nm : k), sizeof(pair_t), cmp_index);
  for (int64_t j = 0; j < k; ++j) {
    if (j < nm) { c->idx[b * k + j] = pr[j].i; if (c->val) c->val[b * k + j] = pr[j].v; }
    else { c->idx[b * k + j] = -1; if (c->val) c->val[b * k + j] = -INFINITY; }
  }
  free(q8); free(qs); free(W); free(s1); free(qd); free(wd); free(key); free(pr);
}

/* Two-stage search.  q: [B, H, d] bf16; w: [B, H]; P: [dc, d]; c: [B, S, dc] int8;
 * cs: [B, S]; k_full: [B, S, d] bf16; nv: [B] or NULL.  Outputs shortlist [B, m],
 * idx [B, k] and val [B, k] (each set in ascending index order), s1 [B, S] or NULL. */
void orc_compact_search(const uint16_t *q, const float *w, const float *P, const int8_t *c, const float *cs,
                        const uint16_t *k_full, const int32_t *nv, int64_t B, int64_t S, int64_t H, int64_t d,
                        int64_t dc, int64_t m, int64_t k, int32_t *shortlist, int32_t *idx, double *val,
                        double *s1) {
  compact_ctx ctx = {q, w, P, c, cs, k_full, nv, S, H, d, dc, m, k, shortlist, idx, val, s1};
  for_rows(B, compact_row, &ctx);
}

/* ---- O4: sparse attention over the selected rows [LC "Stage 2"] --------------------- */

/* q: [Hq, dqk] bf16; rows: [k, dqk] bf16 (row i is kv[idx[i]]); idx: [k] (-1 skipped).
 * out: [Hq, dv], lse: [Hq]. */
static void attn_one(const uint16_t *q, const uint16_t *rows, const int32_t *idx, int64_t Hq, int64_t k,
                     int64_t dqk, int64_t dv, double tau, double *out, double *lse) {
  double *l = (double *)malloc(sizeof(double) * (k > 0 ? k : 1));
  for (int64_t h = 0; h < Hq; ++h) {
    double mx = -INFINITY;
    for (int64_t i = 0; i < k; ++i) {
      if (idx[i] < 0) continue;
      double dot = 0.0;
      for (int64_t j = 0; j < dqk; ++j) dot = fma(orc_dec_bf16(q[h * dqk + j]), orc_dec_bf16(rows[i * dqk + j]), dot);
      l[i] = tau * dot;
      if (l[i] > mx) mx = l[i];
    }
    double den = 0.0;
    for (int64_t j = 0; j < dv; ++j) out[h * dv + j] = 0.0;
    if (mx == -INFINITY) { lse[h] = -INFINITY; continue; }
    for (int64_t i = 0; i < k; ++i) {
      if (idx[i] < 0) continue;
      double e = exp(l[i] - mx);
      den += e;
      for (int64_t j = 0; j < dv; ++j) out[h * dv + j] += e * orc_dec_bf16(rows[i * dqk + j]);
    }
    for (int64_t j = 0; j < dv; ++j) out[h * dv + j] /= den;
    lse[h] = mx + log(den);
  }
  free(l);
}

typedef struct {
  const uint16_t *q; const uint16_t *rows; const int32_t *idx; int64_t Hq, k, dqk, dv; double tau;
  double *out, *lse;
} attn_ctx;

static void attn_row(void *p, int64_t b) {
  attn_ctx *c = (attn_ctx *)p;
  attn_one(c->q + b * c->Hq * c->dqk, c->rows + b * c->k * c->dqk, c->idx + b * c->k, c->Hq, c->k, c->dqk,
           c->dv, c->tau, c->out + b * c->Hq * c->dv, c->lse + b * c->Hq);
}

/* rows: [B, k, dqk], already gathered (row (b, i) = kv[b, idx[b, i]]). */
void orc_sparse_attn_rows(const uint16_t *q, const uint16_t *rows, const int32_t *idx, int64_t B, int64_t Hq,
                          int64_t k, int64_t dqk, int64_t dv, double tau, double *out, double *lse) {
  attn_ctx c = {q, rows, idx, Hq, k, dqk, dv, tau, out, lse};
  for_rows(B, attn_row, &c);
}

/* kv: [B, S, dqk]; gathers the rows named by idx, then attends. */
void orc_sparse_attn(const uint16_t *q, const uint16_t *kv, const int32_t *idx, int64_t B, int64_t Hq,
                     int64_t S, int64_t k, int64_t dqk, int64_t dv, double tau, double *out, double *lse) {
  uint16_t *rows = (uint16_t *)calloc((size_t)(B * k * dqk), sizeof(uint16_t));
  for (int64_t b = 0; b < B; ++b)
    for (int64_t i = 0; i < k; ++i) {
      int32_t s = idx[b * k + i];
      if (s < 0 || s >= S) continue;
      memcpy(rows + (b * k + i) * dqk, kv + (b * S + s) * dqk, sizeof(uint16_t) * dqk);
    }
  orc_sparse_attn_rows(q, rows, idx, B, Hq, k, dqk, dv, tau, out, lse);
  free(rows);
}

/* ---- O6: pooled indexer keys (IndexPool) ["Long context", section "The 2025-2026
 * Hybrid Turn: Linear Attention Returns", GLM-5.3-Flash: four indexer keys pooled
 * into one, index_kpool = 4; "Latent Sparse Attention", section "Where the time
 * goes": 32 heads x 128 dims scoring keys pooled four at a time, top-512 blocks] --- */

/* Nearest OCP E4M3FN value to x (finite), ties to the even code, saturating at
 * +-448: the non-negative finite codes 0x00..0x7E decode to ascending values, so
 * a binary search finds the two codes around |x| and the nearer one wins, the
 * even one on a tie. */
uint8_t orc_e4m3_rne(float x) {
  double a = fabs((double)x);
  uint8_t best;
  if (a >= 448.0) {
    best = 0x7E;
  } else {
    int lo = 0, hi = 0x7E; /* invariant: value(lo) <= a < value(hi) */
    while (hi - lo > 1) {
      int mid = (lo + hi) / 2;
      if (orc_dec_e4m3((uint8_t)mid) <= a) lo = mid; else hi = mid;
    }
    double dl = a - orc_dec_e4m3((uint8_t)lo), dh = orc_dec_e4m3((uint8_t)hi) - a;
    best = (uint8_t)(dl < dh ? lo : dh < dl ? hi : ((lo & 1) == 0 ? lo : hi));
  }
  return (uint8_t)(best | (signbit(x) ? 0x80 : 0x00));
}

/* Pool `pool` consecutive bf16 token keys into one fp8 key with an fp32 scale (the
 * pooled cache is written when a block of `pool` tokens completes; an incomplete
 * last block is not pooled).  The pooled value is the mean: m_j = (((k_0 + k_1) +
 * k_2) + ...) * (1 / pool) in fp32 (pool a power of two, so the scaling is exact);
 * scale = max_j |m_j| / 448 (fp32, 1 if all are zero); code_j = e4m3_rne(m_j /
 * scale) (fp32 division).  These steps decide integer codes, so they are taken in
 * the fp32 arithmetic the kernel uses, in this order.
 * k: [B, L, d] bf16 -> codes [B, L / pool, d], scales [B, L / pool]. */
void orc_pool_keys(const uint16_t *k, int64_t B, int64_t L, int64_t d, int64_t pool, uint8_t *codes,
                   float *scales) {
  int64_t Sp = L / pool;
  float *m = (float *)malloc(sizeof(float) * (d > 0 ? d : 1));
  for (int64_t b = 0; b < B; ++b)
    for (int64_t j = 0; j < Sp; ++j) {
      float amax = 0.0f;
      for (int64_t i = 0; i < d; ++i) {
        float s = (float)orc_dec_bf16(k[(b * L + j * pool) * d + i]);
        for (int64_t t = 1; t < pool; ++t) s = s + (float)orc_dec_bf16(k[(b * L + j * pool + t) * d + i]);
        m[i] = s * (1.0f / (float)pool);
        if (fabsf(m[i]) > amax) amax = fabsf(m[i]);
      }
      float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
      scales[b * Sp + j] = sc;
      for (int64_t i = 0; i < d; ++i) codes[(b * Sp + j) * d + i] = orc_e4m3_rne(m[i] / sc);
    }
  free(m);
}

/* Selection over pooled keys, expanded to tokens: score every complete visible
 * block (nv_tokens[r] / pool of them, at most Sp) with the indexer score (O1 on
 * the fp8 pooled keys), take the top-k blocks (O2), and list each selected block
 * j as its tokens pool * j .. pool * j + pool - 1; a padded block (-1) gives pool
 * entries of -1.  idx_tokens: [B*T, k * pool] in ascending token order; val_blocks:
 * [B*T, k] or NULL, the selected blocks' scores.  nv_tokens NULL = every block. */
void orc_pooled_select(const void *q, int q_type, const float *w, const uint8_t *codes, const float *scales,
                       const int32_t *nv_tokens, int64_t B, int64_t T, int64_t Sp, int64_t H, int64_t d,
                       int64_t pool, int64_t k, int32_t *idx_tokens, double *val_blocks) {
  int64_t R = B * T;
  int32_t *nvb = (int32_t *)malloc(sizeof(int32_t) * (R > 0 ? R : 1));
  for (int64_t r = 0; r < R; ++r) {
    int64_t n = nv_tokens ? (int64_t)nv_tokens[r] / pool : Sp;
    if (nv_tokens && nv_tokens[r] < 0) n = 0;
    nvb[r] = (int32_t)(n < Sp ? n : Sp);
  }
  double *sc = (double *)malloc(sizeof(double) * (R * Sp > 0 ? R * Sp : 1));
  orc_indexer_score(q, q_type, w, codes, ORC_FP8_E4M3, scales, nvb, B, T, Sp, H, d, sc);
  int32_t *blk = (int32_t *)malloc(sizeof(int32_t) * (R * k > 0 ? R * k : 1));
  orc_topk(sc, nvb, R, Sp, k, blk, val_blocks);
  for (int64_t r = 0; r < R; ++r)
    for (int64_t j = 0; j < k; ++j)
      for (int64_t t = 0; t < pool; ++t) {
        int32_t bj = blk[r * k + j];
        idx_tokens[(r * k + j) * pool + t] = bj < 0 ? -1 : (int32_t)(bj * pool + t);
      }
  free(nvb); free(sc); free(blk);
}

/* ---- O7: product-quantised compact keys [LS 07:12-08:00: each 128-d key split
 * into 32 four-dimension pieces, each piece a one-byte index into a 256-entry
 * codebook trained offline; a coarse pass over the codes keeps 2,048 candidates,
 * their original keys are reranked exactly to 512] ----------------------------- */

/* Query side for one (b, h): q8 = rint(q / qs) clamped to [-127, 127] with
 * qs = max|q| / 127 (1 if zero), W = (w * qs) * sigma, all in fp64. */
static void pq_query_one(const uint16_t *q, float w, double sigma, int64_t d, int8_t *q8, double *W) {
  double amax = 0.0;
  for (int64_t i = 0; i < d; ++i) {
    double v = fabs(orc_dec_bf16(q[i]));
    if (v > amax) amax = v;
  }
  double qs = amax > 0.0 ? amax / 127.0 : 1.0;
  for (int64_t i = 0; i < d; ++i) {
    double t = rint(orc_dec_bf16(q[i]) / qs);
    if (t > 127.0) t = 127.0;
    if (t < -127.0) t = -127.0;
    q8[i] = (int8_t)t;
  }
  *W = ((double)w * qs) * sigma;
}

/* q: [B, H, d] bf16 -> q8 [B, H, d] int8, W [B, H] fp64. */
void orc_pq_query(const uint16_t *q, const float *w, double sigma, int64_t B, int64_t H, int64_t d, int8_t *q8,
                  double *W) {
  for (int64_t r = 0; r < B * H; ++r) pq_query_one(q + r * d, w[r], sigma, d, q8 + r * d, W + r);
}

/* Stage-1 score of one key from its codes: the key is decoded piece by piece from
 * the codebook, D_h = q8_h . decoded key (exact integers), and
 * s1 = chain_h(W_h, max(D_h, 0)) (fp64 fma chain, h ascending). */
static double pq_stage1_one(const int8_t *q8, const double *W, const uint8_t *code, const int8_t *cb, int64_t H,
                            int64_t d) {
  int64_t np = d / 4;
  double acc = 0.0;
  for (int64_t h = 0; h < H; ++h) {
    int64_t D = 0;
    for (int64_t j = 0; j < np; ++j) {
      const int8_t *c = cb + (j * 256 + code[j]) * 4;
      for (int64_t i = 0; i < 4; ++i) D += (int64_t)q8[h * d + 4 * j + i] * (int64_t)c[i];
    }
    acc = fma(W[h], (double)(D > 0 ? D : 0), acc);
  }
  return acc;
}

typedef struct {
  const uint16_t *q; const float *w; const int8_t *cb; double sigma; const uint8_t *codes;
  const uint16_t *kf; const int32_t *nv; int64_t S, H, d, m, k;
  int32_t *shortlist; int32_t *idx; double *val; double *s1_out;
} pq_ctx;

static void pq_row(void *p, int64_t b) {
  pq_ctx *c = (pq_ctx *)p;
  int64_t S = c->S, H = c->H, d = c->d, m = c->m, k = c->k, np = d / 4;
  int8_t *q8 = (int8_t *)malloc((size_t)(H * d));
  double *W = (double *)malloc(sizeof(double) * H);
  for (int64_t h = 0; h < H; ++h)
    pq_query_one(c->q + (b * H + h) * d, c->w[b * H + h], c->sigma, d, q8 + h * d, W + h);
  int64_t nv = c->nv ? c->nv[b] : S;
  if (nv > S) nv = S;
  if (nv < 0) nv = 0;
  double *s1 = (double *)malloc(sizeof(double) * (nv > 0 ? nv : 1));
  for (int64_t s = 0; s < nv; ++s) s1[s] = pq_stage1_one(q8, W, c->codes + (b * S + s) * np, c->cb, H, d);
  if (c->s1_out)
    for (int64_t s = 0; s < S; ++s) c->s1_out[b * S + s] = s < nv ? s1[s] : -INFINITY;
  int32_t *sl = c->shortlist + b * m;
  topk_one(s1, nv, m, sl, NULL);
  /* stage 2: the exact score of the shortlisted original keys, keep the top k */
  double *qd = (double *)malloc(sizeof(double) * H * d);
  double *wd = (double *)malloc(sizeof(double) * H);
  double *key = (double *)malloc(sizeof(double) * d);
  for (int64_t i = 0; i < H * d; ++i) qd[i] = orc_dec_bf16(c->q[b * H * d + i]);
  for (int64_t h = 0; h < H; ++h) wd[h] = (double)c->w[b * H + h];
  int64_t nm = nv < m ? nv : m;
  pair_t *pr = (pair_t *)malloc(sizeof(pair_t) * (nm > 0 ? nm : 1));
  for (int64_t i = 0; i < nm; ++i) {
    int64_t s = sl[i];
    for (int64_t j = 0; j < d; ++j) key[j] = orc_dec_bf16(c->kf[(b * S + s) * d + j]);
    pr[i].v = score_one(qd, wd, key, H, d);
    pr[i].i = (int32_t)s;
  }
  qsort(pr, (size_t)nm, sizeof(pair_t), cmp_desc);
  qsort(pr, (size_t)(nm < k ? nm : k), sizeof(pair_t), cmp_index);
  for (int64_t j = 0; j < k; ++j) {
    if (j < nm) { c->idx[b * k + j] = pr[j].i; if (c->val) c->val[b * k + j] = pr[j].v; }
    else { c->idx[b * k + j] = -1; if (c->val) c->val[b * k + j] = -INFINITY; }
  }
  free(q8); free(W); free(s1); free(qd); free(wd); free(key); free(pr);
}

/* Two-stage search over product-quantised keys.  q: [B, H, d] bf16; w: [B, H];
 * cb: [d / 4, 256, 4] int8 codebook entries (piece j of code c is
 * sigma * cb[j, c, :]); codes: [B, S, d / 4] uint8; k_full: [B, S, d] bf16;
 * nv: [B] or NULL.  Outputs shortlist [B, m], idx [B, k], val [B, k] (ascending
 * index order), s1 [B, S] or NULL. */
void orc_pq_search(const uint16_t *q, const float *w, const int8_t *cb, double sigma, const uint8_t *codes,
                   const uint16_t *k_full, const int32_t *nv, int64_t B, int64_t S, int64_t H, int64_t d, int64_t m,
                   int64_t k, int32_t *shortlist, int32_t *idx, double *val, double *s1) {
  pq_ctx ctx = {q, w, cb, sigma, codes, k_full, nv, S, H, d, m, k, shortlist, idx, val, s1};
  for_rows(B, pq_row, &ctx);
}

