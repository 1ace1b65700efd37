/*
 * Host-only driver for an AddressSanitizer + UndefinedBehaviorSanitizer run of the
 * CPU oracle (oracle/oracle.c) and the input generator (synth/gen.c).  Built and
 * run by tests/test_sanitize.py with gcc; it calls every exported function of both
 * files on small inputs, including the edge cases (no visible key, fewer visible
 * keys than k, skipped attention rows, k larger than the row, one thread and
 * several), and exits 0 when every call returned.  The sanitizers abort the run on
 * the first out-of-bounds access, leak or undefined operation.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

/* oracle/oracle.c */
double orc_dec_bf16(uint16_t b);
double orc_dec_e4m3(uint8_t c);
int orc_threads_used(void);
void orc_indexer_score(const void *q, int q_type, const float *w, const void *k, int k_type, const float *k_scale,
                       const int32_t *nv, int64_t B, int64_t T, int64_t S, int64_t H, int64_t d, double *scores);
void orc_topk(const double *scores, const int32_t *nv, int64_t R, int64_t S, int64_t k, int32_t *idx, double *val);
void orc_compact_query(const uint16_t *q, const float *w, const float *P, int64_t B, int64_t H, int64_t d, int64_t dc,
                       int8_t *q8, double *qs, double *W);
void orc_compact_search(const uint16_t *q, const float *w, const float *P, const int8_t *c, const float *cs,
                        const uint16_t *k_full, const int32_t *nv, int64_t B, int64_t S, int64_t H, int64_t d,
                        int64_t dc, int64_t m, int64_t k, int32_t *shortlist, int32_t *idx, double *val, double *s1);
void orc_sparse_attn_rows(const uint16_t *q, const uint16_t *rows, const int32_t *idx, int64_t B, int64_t Hq,
                          int64_t k, int64_t dqk, int64_t dv, double tau, double *out, double *lse);
void orc_sparse_attn(const uint16_t *q, const uint16_t *kv, const int32_t *idx, int64_t B, int64_t Hq, int64_t S,
                     int64_t k, int64_t dqk, int64_t dv, double tau, double *out, double *lse);

uint8_t orc_e4m3_rne(float x);
void orc_pool_keys(const uint16_t *k, int64_t B, int64_t L, int64_t d, int64_t pool, uint8_t *codes, float *scales);
void orc_pooled_select(const void *q, int q_type, const float *w, const uint8_t *codes, const float *scales,
                       const int32_t *nv_tokens, int64_t B, int64_t T, int64_t Sp, int64_t H, int64_t d,
                       int64_t pool, int64_t k, int32_t *idx_tokens, double *val_blocks);

void orc_pq_query(const uint16_t *q, const float *w, double sigma, int64_t B, int64_t H, int64_t d, int8_t *q8,
                  double *W);
void orc_pq_search(const uint16_t *q, const float *w, const int8_t *cb, double sigma, const uint8_t *codes,
                   const uint16_t *k_full, const int32_t *nv, int64_t B, int64_t S, int64_t H, int64_t d, int64_t m,
                   int64_t k, int32_t *shortlist, int32_t *idx, double *val, double *s1);

/* synth/gen.c */
uint64_t synth_stream_base(uint64_t seed, uint64_t tid);
uint16_t synth_bf16_rne(double v);
uint8_t synth_e4m3_rne(double v);
void synth_normal_f64(uint64_t seed, uint64_t tid, uint64_t off, uint64_t n, double scale, double *out);
void synth_normal_f32(uint64_t seed, uint64_t tid, uint64_t off, uint64_t n, double scale, float *out);
void synth_normal_bf16(uint64_t seed, uint64_t tid, uint64_t off, uint64_t n, double scale, uint16_t *out);
void synth_uniform_f32(uint64_t seed, uint64_t tid, uint64_t off, uint64_t n, double lo, double hi, float *out);
void synth_uniform_f64(uint64_t seed, uint64_t tid, uint64_t off, uint64_t n, double lo, double hi, double *out);
void synth_normal_bf16_rows(uint64_t seed, uint64_t tid, const int64_t *rows, uint64_t nrows, uint64_t d,
                            double scale, uint16_t *out);
void synth_fp8_rows(uint64_t seed, uint64_t tid, uint64_t row_off, uint64_t rows, uint64_t d, double scale,
                    uint8_t *codes, float *scales);
void synth_compact_keys(const uint16_t *k_bf16, uint64_t rows, uint64_t d, const float *P, uint64_t dc, int8_t *c,
                        float *cs);
int synth_threads(void);
void synth_pq_codebook(const uint16_t *k, uint64_t n, uint64_t d, uint64_t seed, int iters, int8_t *cb,
                       float *sigma);
void synth_pq_encode(const uint16_t *k, uint64_t rows, uint64_t d, const int8_t *cb, float sigma, uint8_t *codes);

enum { F32 = 0, BF16 = 1, FP8 = 2 };

static void *xmalloc(size_t n) {
  void *p = malloc(n ? n : 1);
  if (!p) {
    fprintf(stderr, "out of memory\n");
    exit(2);
  }
  return p;
}

int main(void) {
  const int64_t B = 2, T = 3, S = 97, H = 5, d = 128, dc = 32;
  /* generator: every entry point */
  (void)synth_stream_base(1, 2);
  double special[] = {0.0, -0.0, 1e-40, 448.0, 500.0, -1e30, 3.14159, NAN, INFINITY};
  for (size_t i = 0; i < sizeof special / sizeof special[0]; ++i) {
    (void)synth_bf16_rne(special[i]);
    (void)synth_e4m3_rne(special[i]);
  }
  double *f64 = xmalloc(sizeof(double) * 1001);
  float *f32 = xmalloc(sizeof(float) * 1001);
  synth_normal_f64(7, 1, 3, 1001, 1.0, f64);
  synth_normal_f32(7, 1, 0, 1001, 0.5, f32);
  synth_uniform_f64(7, 2, 0, 1001, -1.0, 1.0, f64);
  uint16_t *qb = xmalloc(sizeof(uint16_t) * B * T * H * d);
  synth_normal_bf16(7, 3, 0, (uint64_t)(B * T * H * d), 0.1, qb);
  float *w = xmalloc(sizeof(float) * B * T * H);
  synth_uniform_f32(7, 4, 0, (uint64_t)(B * T * H), 0.0, 1.0, w);
  uint8_t *k8 = xmalloc((size_t)(B * S * d));
  float *ks = xmalloc(sizeof(float) * B * S);
  synth_fp8_rows(7, 5, 0, (uint64_t)(B * S), (uint64_t)d, 1.0, k8, ks);
  uint16_t *kb = xmalloc(sizeof(uint16_t) * B * S * d);
  synth_normal_bf16(7, 6, 0, (uint64_t)(B * S * d), 1.0, kb);
  int64_t rows[] = {0, 5, 96, 150};
  uint16_t *rb = xmalloc(sizeof(uint16_t) * 4 * d);
  synth_normal_bf16_rows(7, 6, rows, 4, (uint64_t)d, 1.0, rb);
  float *P = xmalloc(sizeof(float) * dc * d);
  synth_normal_f32(7, 7, 0, (uint64_t)(dc * d), 0.17, P);
  int8_t *ck = xmalloc((size_t)(B * S * dc));
  float *cks = xmalloc(sizeof(float) * B * S);
  synth_compact_keys(kb, (uint64_t)(B * S), (uint64_t)d, P, (uint64_t)dc, ck, cks);
  (void)synth_threads();

  /* oracle: decoders over every code */
  double acc = 0.0;
  for (int c = 0; c < 256; ++c) acc += isnan(orc_dec_e4m3((uint8_t)c)) ? 0.0 : orc_dec_e4m3((uint8_t)c);
  for (int c = 0; c < 65536; c += 7) acc += isfinite(orc_dec_bf16((uint16_t)c)) ? 0.0 : 1.0;

  /* scores with and without a visibility vector (0, below k, S, beyond S) */
  int32_t nv[6] = {0, 3, 97, 200, 50, 1};
  double *sc = xmalloc(sizeof(double) * B * T * S);
  orc_indexer_score(qb, BF16, w, k8, FP8, ks, nv, B, T, S, H, d, sc);
  orc_indexer_score(qb, BF16, w, kb, BF16, NULL, NULL, B, T, S, H, d, sc);
  orc_indexer_score(f32, F32, w, f32, F32, NULL, NULL, 1, 1, 7, 1, d, sc);
  (void)orc_threads_used();

  /* top-k: k below, at and above the visible count */
  const int64_t ks_[] = {1, 8, 97, 150};
  for (size_t i = 0; i < sizeof ks_ / sizeof ks_[0]; ++i) {
    int64_t kk = ks_[i];
    int32_t *idx = xmalloc(sizeof(int32_t) * B * T * kk);
    double *val = xmalloc(sizeof(double) * B * T * kk);
    orc_topk(sc, nv, B * T, S, kk, idx, val);
    orc_topk(sc, NULL, B * T, S, kk, idx, NULL);
    free(idx);
    free(val);
  }

  /* compact search: m and k up to and past the visible count */
  uint16_t *qc = xmalloc(sizeof(uint16_t) * B * H * d);
  synth_normal_bf16(7, 8, 0, (uint64_t)(B * H * d), 0.1, qc);
  float *wc = xmalloc(sizeof(float) * B * H);
  synth_uniform_f32(7, 9, 0, (uint64_t)(B * H), 0.0, 1.0, wc);
  int8_t *q8 = xmalloc((size_t)(B * H * dc));
  double *qs = xmalloc(sizeof(double) * B * H), *W = xmalloc(sizeof(double) * B * H);
  orc_compact_query(qc, wc, P, B, H, d, dc, q8, qs, W);
  int32_t cnv[2] = {10, 97};
  const int64_t mk[][2] = {{16, 4}, {97, 97}, {120, 100}};
  for (size_t i = 0; i < 3; ++i) {
    int64_t m = mk[i][0], kk = mk[i][1];
    int32_t *sl = xmalloc(sizeof(int32_t) * B * m), *fi = xmalloc(sizeof(int32_t) * B * kk);
    double *fv = xmalloc(sizeof(double) * B * kk), *s1 = xmalloc(sizeof(double) * B * S);
    orc_compact_search(qc, wc, P, ck, cks, kb, cnv, B, S, H, d, dc, m, kk, sl, fi, fv, s1);
    orc_compact_search(qc, wc, P, ck, cks, kb, NULL, B, S, H, d, dc, m, kk, sl, fi, NULL, NULL);
    free(sl); free(fi); free(fv); free(s1);
  }

  /* sparse attention: skipped rows, all rows skipped, repeated rows */
  const int64_t Hq = 3, dqk = 24, dv = 16, ka = 6;
  uint16_t *qa = xmalloc(sizeof(uint16_t) * B * Hq * dqk), *kv = xmalloc(sizeof(uint16_t) * B * S * dqk);
  synth_normal_bf16(7, 10, 0, (uint64_t)(B * Hq * dqk), 1.0, qa);
  synth_normal_bf16(7, 11, 0, (uint64_t)(B * S * dqk), 1.0, kv);
  int32_t ia[12] = {0, 96, -1, 5, 5, 40, -1, -1, -1, -1, -1, -1};
  double *out = xmalloc(sizeof(double) * B * Hq * dv), *lse = xmalloc(sizeof(double) * B * Hq);
  orc_sparse_attn(qa, kv, ia, B, Hq, S, ka, dqk, dv, 0.2, out, lse);
  uint16_t *gathered = xmalloc(sizeof(uint16_t) * B * ka * dqk);
  memset(gathered, 0, sizeof(uint16_t) * B * ka * dqk);
  orc_sparse_attn_rows(qa, gathered, ia, B, Hq, ka, dqk, dv, 0.2, out, lse);

  /* pooled keys: an incomplete last block, visible counts below one block */
  for (int c = -500; c <= 500; c += 3) (void)orc_e4m3_rne((float)c * 0.917f);
  const int64_t pool = 4, Sp = S / pool, kp = 5;
  uint8_t *pc = xmalloc((size_t)(B * Sp * d));
  float *ps = xmalloc(sizeof(float) * B * Sp);
  orc_pool_keys(kb, B, S, d, pool, pc, ps);
  int32_t pnv[6] = {0, 3, 4, 97, 1000, 23};
  int32_t *pidx = xmalloc(sizeof(int32_t) * B * T * kp * pool);
  double *pval = xmalloc(sizeof(double) * B * T * kp);
  orc_pooled_select(qb, BF16, w, pc, ps, pnv, B, T, Sp, H, d, pool, kp, pidx, pval);
  int32_t *pidx2 = xmalloc(sizeof(int32_t) * B * T * 40 * pool); /* k above the block count */
  orc_pooled_select(qb, BF16, w, pc, ps, NULL, B, T, Sp, H, d, pool, 40, pidx2, NULL);
  free(pc); free(ps); free(pidx); free(pval); free(pidx2);

  /* product-quantised keys: codebooks from fewer keys than entries, codes, search */
  int8_t *cb = xmalloc(32 * 256 * 4);
  float sigma = 0.0f;
  synth_pq_codebook(kb, (uint64_t)(B * S), (uint64_t)d, 7, 3, cb, &sigma);
  uint8_t *pqc = xmalloc((size_t)(B * S * 32));
  synth_pq_encode(kb, (uint64_t)(B * S), (uint64_t)d, cb, sigma, pqc);
  int8_t *pq8 = xmalloc((size_t)(B * H * d));
  double *pW = xmalloc(sizeof(double) * B * H);
  orc_pq_query(qc, wc, sigma, B, H, d, pq8, pW);
  for (size_t i = 0; i < 3; ++i) {
    int64_t m = mk[i][0], kk = mk[i][1];
    int32_t *sl = xmalloc(sizeof(int32_t) * B * m), *fi = xmalloc(sizeof(int32_t) * B * kk);
    double *fv = xmalloc(sizeof(double) * B * kk), *s1 = xmalloc(sizeof(double) * B * S);
    orc_pq_search(qc, wc, cb, sigma, pqc, kb, cnv, B, S, H, d, m, kk, sl, fi, fv, s1);
    orc_pq_search(qc, wc, cb, sigma, pqc, kb, NULL, B, S, H, d, m, kk, sl, fi, NULL, NULL);
    free(sl); free(fi); free(fv); free(s1);
  }
  free(cb); free(pqc); free(pq8); free(pW);

  free(f64); free(f32); free(qb); free(w); free(k8); free(ks); free(kb); free(rb); free(P); free(ck); free(cks);
  free(sc); free(qc); free(wc); free(q8); free(qs); free(W); free(qa); free(kv); free(out); free(lse);
  free(gathered);
  printf("sanitized run ok (%g)\n", acc);
  return 0;
}
