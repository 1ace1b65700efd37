/*
 * Seeded synthetic inputs for the lightning-indexer workloads.
 *
 * This file is input plumbing only: random draws and the storage formats the
 * inputs are kept in (fp32, bf16, fp8 E4M3FN with a per-row fp32 scale, and the
 * int8 compact-key encoding).  It computes no score, selection or attention.
 *
 * Random numbers come from splitmix64 in counter mode (Steele, Lea and Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014): the stream of
 * tensor `tid` under seed `seed` has state base = mix(mix(seed) + tid * GAMMA),
 * and its i-th 64-bit output is mix(base + (i + 1) * GAMMA).  Any element of any
 * tensor can therefore be regenerated alone from (seed, tid, flat index), which
 * lets a checker rebuild only the rows it needs out of a multi-GiB tensor.
 *
 * Normals use the Box-Muller transform on a pair of outputs: element i takes
 * pair p = i / 2, u1 = ((r[2p] >> 11) + 1) * 2^-53 in (0, 1],
 * u2 = (r[2p+1] >> 11) * 2^-53 in [0, 1), radius sqrt(-2 ln u1), angle 2 pi u2,
 * and the cosine for even i, the sine for odd i.
 *
 * Keys stored in fp8 follow the key-cache format of the "Long context" lecture
 * (llm-serving.xyz lecture 03), section "The Architectural Answer", paragraph
 * "Stage 1, the lightning indexer": a 128-byte FP8 key plus a 4-byte scale.
 * Here the scale is rowmax|x| / 448 rounded to fp32 (1 for an all-zero row) and
 * each code is x / scale rounded to nearest-even in OCP E4M3FN, saturated at 448.
 *
 * Compact keys (a fixed random Gaussian 128 -> 32 projection, int8 with a per-row
 * fp32 scale) stand in for the compact indexer keys of the LeanSparse podcast
 * transcript (cues 07:12-07:34): y = P k in fp64 with an fma chain over the key
 * dimension in ascending order, scale = max|y| / 127 rounded to fp32 (1 for an
 * all-zero row), code = clamp(rint(y / scale), -127, 127).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

uint64_t synth_stream_base(uint64_t seed, uint64_t tid) {
  return mix64(mix64(seed) + tid * GAMMA);
}

static inline uint64_t draw(uint64_t base, uint64_t i) {
  return mix64(base + (i + 1) * GAMMA);
}

static const double TWO_PI = 6.283185307179586476925286766559;

/* Normal pair for pair index p: (cos branch, sin branch). */
static inline void normal_pair(uint64_t base, uint64_t p, double *z0, double *z1) {
  uint64_t r1 = draw(base, 2 * p), r2 = draw(base, 2 * p + 1);
  double u1 = (double)((r1 >> 11) + 1) * 0x1.0p-53;
  double u2 = (double)(r2 >> 11) * 0x1.0p-53;
  double rad = sqrt(-2.0 * log(u1));
  double th = TWO_PI * u2;
  *z0 = rad * cos(th);
  *z1 = rad * sin(th);
}

static inline double normal_at(uint64_t base, uint64_t i) {
  double z0, z1;
  normal_pair(base, i >> 1, &z0, &z1);
  return (i & 1) ? z1 : z0;
}

static inline double uniform_at(uint64_t base, uint64_t i) {
  return (double)(draw(base, i) >> 11) * 0x1.0p-53;
}

/* ---- storage-format encoders ------------------------------------------ */

/* fp64 -> bf16 bits, round to nearest even: round to odd into fp32 first
 * (fp32 keeps 16 more significand bits than bf16, so the final RNE step sees
 * an exact sticky bit), then round fp32 -> bf16 to nearest even. */
uint16_t synth_bf16_rne(double v) {
  float f = (float)v;
  if ((double)f != v && !isnan(v) && !isinf(f)) {
    if (fabs((double)f) > fabs(v)) f = nextafterf(f, 0.0f);
    uint32_t u;
    memcpy(&u, &f, 4);
    u |= 1u;
    memcpy(&f, &u, 4);
  }
  uint32_t u;
  memcpy(&u, &f, 4);
  if (isnan(f)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* fp64 -> OCP fp8 E4M3FN code (bias 7, 3 mantissa bits, max 448, no inf),
 * round to nearest even, saturating at +-448. */
uint8_t synth_e4m3_rne(double v) {
  uint8_t sign = (v < 0.0 || (v == 0.0 && signbit(v))) ? 0x80 : 0x00;
  double a = fabs(v);
  if (!(a < 448.0)) return sign | 0x7E; /* saturate (NaN inputs are not produced) */
  if (a < 0x1.0p-6) {
    /* subnormal range: value = n * 2^-9 with n in [0, 8]; n = 8 is the
     * smallest normal (exponent field 1, mantissa 0), which the same
     * integer encodes */
    int n = (int)rint(a * 512.0);
    return sign | (uint8_t)n;
  }
  /* normal range: keep 3 fraction bits of the fp64 significand, round to
   * nearest even; a carry out of the fraction bumps the exponent field */
  uint64_t b;
  memcpy(&b, &a, 8);
  uint64_t keep = b >> 49;                 /* sign(0) | exp11 | frac3 */
  uint64_t rest = b & ((1ULL << 49) - 1);
  uint64_t half = 1ULL << 48;
  if (rest > half || (rest == half && (keep & 1))) keep += 1;
  int e = (int)(keep >> 3) - 1023;         /* unbiased exponent after rounding */
  int m = (int)(keep & 7);
  if (e > 8 || (e == 8 && m > 6)) return sign | 0x7E;
  return sign | (uint8_t)(((e + 7) << 3) | m);
}

/* ---- threading ----------------------------------------------------------- */

typedef void (*range_fn)(void *ctx, uint64_t lo, uint64_t hi);
typedef struct { range_fn fn; void *ctx; uint64_t lo, hi; } job_t;

static void *job_run(void *p) {
  job_t *j = (job_t *)p;
  j->fn(j->ctx, j->lo, j->hi);
  return NULL;
}

static int n_threads(void) {
  const char *s = getenv("SYNTH_THREADS");
  long n = s ? atol(s) : sysconf(_SC_NPROCESSORS_ONLN);
  if (n < 1) n = 1;
  if (n > 16) n = 16;
  return (int)n;
}

/* Split [0, n) in `grain`-aligned chunks over threads; results do not depend on
 * the split because every element is a pure function of its index. */
static void parallel_for(uint64_t n, uint64_t grain, range_fn fn, void *ctx) {
  int nt = n_threads();
  uint64_t units = (n + grain - 1) / grain;
  if (units < (uint64_t)nt) nt = (int)(units ? units : 1);
  if (nt <= 1) { fn(ctx, 0, n); return; }
  pthread_t th[32];
  job_t jobs[32];
  uint64_t per = (units + nt - 1) / nt;
  int used = 0;
  for (int t = 0; t < nt; ++t) {
    uint64_t lo = (uint64_t)t * per * grain, hi = lo + per * grain;
    if (lo >= n) break;
    if (hi > n) hi = n;
    jobs[t] = (job_t){fn, ctx, lo, hi};
    pthread_create(&th[t], NULL, job_run, &jobs[t]);
    used++;
  }
  for (int t = 0; t < used; ++t) pthread_join(th[t], NULL);
}

/* ---- dense tensors --------------------------------------------------------- */

typedef struct {
  uint64_t base, off;
  double scale, lo, hi;
  void *out;
  int kind; /* 0 f64 normal, 1 f32 normal, 2 bf16 normal, 3 f32 uniform, 4 f64 uniform */
} dense_ctx;

static void dense_range(void *p, uint64_t lo, uint64_t hi) {
  dense_ctx *c = (dense_ctx *)p;
  for (uint64_t i = lo; i < hi; ++i) {
    uint64_t g = c->off + i;
    switch (c->kind) {
      case 0: ((double *)c->out)[i] = c->scale * normal_at(c->base, g); break;
      case 1: ((float *)c->out)[i] = (float)(c->scale * normal_at(c->base, g)); break;
      case 2: ((uint16_t *)c->out)[i] = synth_bf16_rne(c->scale * normal_at(c->base, g)); break;
      case 3: ((float *)c->out)[i] = (float)(c->lo + (c->hi - c->lo) * uniform_at(c->base, g)); break;
      case 4: ((double *)c->out)[i] = c->lo + (c->hi - c->lo) * uniform_at(c->base, g); break;
    }
  }
}

/* bf16 normals are the bulk of the large tensors: generate them pairwise. */
static void bf16_pair_range(void *p, uint64_t lo, uint64_t hi) {
  dense_ctx *c = (dense_ctx *)p;
  uint16_t *o = (uint16_t *)c->out;
  uint64_t i = lo;
  while (i < hi) {
    uint64_t g = c->off + i;
    if ((g & 1) == 0 && i + 1 < hi) {
      double z0, z1;
      normal_pair(c->base, g >> 1, &z0, &z1);
      o[i] = synth_bf16_rne(c->scale * z0);
      o[i + 1] = synth_bf16_rne(c->scale * z1);
      i += 2;
    } else {
      o[i] = synth_bf16_rne(c->scale * normal_at(c->base, g));
      i += 1;
    }
  }
}

static void dense(uint64_t seed, uint64_t tid, uint64_t off, uint64_t n, int kind,
                  double scale, double lo, double hi, void *out) {
  dense_ctx c = {synth_stream_base(seed, tid), off, scale, lo, hi, out, kind};
  parallel_for(n, 4096, kind == 2 ? bf16_pair_range : dense_range, &c);
}

void synth_normal_f64(uint64_t seed, uint64_t tid, uint64_t off, uint64_t n, double scale, double *out) {
  dense(seed, tid, off, n, 0, scale, 0, 0, out);
}
void synth_normal_f32(uint64_t seed, uint64_t tid, uint64_t off, uint64_t n, double scale, float *out) {
  dense(seed, tid, off, n, 1, scale, 0, 0, out);
}
void synth_normal_bf16(uint64_t seed, uint64_t tid, uint64_t off, uint64_t n, double scale, uint16_t *out) {
  dense(seed, tid, off, n, 2, scale, 0, 0, out);
}
void synth_uniform_f32(uint64_t seed, uint64_t tid, uint64_t off, uint64_t n, double lo, double hi, float *out) {
  dense(seed, tid, off, n, 3, 1.0, lo, hi, out);
}
void synth_uniform_f64(uint64_t seed, uint64_t tid, uint64_t off, uint64_t n, double lo, double hi, double *out) {
  dense(seed, tid, off, n, 4, 1.0, lo, hi, out);
}

/* Gather rows [rows[i], :] of a bf16-normal tensor with row length `d` (so a
 * checker can rebuild selected rows of a tensor too large to regenerate). */
typedef struct { uint64_t base; const int64_t *rows; uint64_t d; double scale; uint16_t *out; } rows_ctx;
static void rows_range(void *p, uint64_t lo, uint64_t hi) {
  rows_ctx *c = (rows_ctx *)p;
  for (uint64_t r = lo; r < hi; ++r) {
    uint64_t g0 = (uint64_t)c->rows[r] * c->d;
    for (uint64_t j = 0; j < c->d; ++j)
      c->out[r * c->d + j] = synth_bf16_rne(c->scale * normal_at(c->base, g0 + j));
  }
}
void synth_normal_bf16_rows(uint64_t seed, uint64_t tid, const int64_t *rows, uint64_t nrows,
                            uint64_t d, double scale, uint16_t *out) {
  rows_ctx c = {synth_stream_base(seed, tid), rows, d, scale, out};
  parallel_for(nrows, 16, rows_range, &c);
}

/* ---- fp8 E4M3FN rows with a per-row fp32 scale ------------------------------ */

typedef struct { uint64_t base, row_off, d; double scale; uint8_t *codes; float *scales; } fp8_ctx;

static void fp8_range(void *p, uint64_t lo, uint64_t hi) {
  fp8_ctx *c = (fp8_ctx *)p;
  double *x = (double *)malloc(sizeof(double) * (c->d + 1));
  for (uint64_t r = lo; r < hi; ++r) {
    uint64_t g0 = (c->row_off + r) * c->d;
    double amax = 0.0;
    uint64_t j = 0;
    while (j < c->d) {
      uint64_t g = g0 + j;
      if ((g & 1) == 0 && j + 1 < c->d) {
        double z0, z1;
        normal_pair(c->base, g >> 1, &z0, &z1);
        x[j] = c->scale * z0;
        x[j + 1] = c->scale * z1;
        j += 2;
      } else {
        x[j] = c->scale * normal_at(c->base, g);
        j += 1;
      }
    }
    for (j = 0; j < c->d; ++j)
      if (fabs(x[j]) > amax) amax = fabs(x[j]);
    float sc = amax > 0.0 ? (float)(amax / 448.0) : 1.0f;
    c->scales[r] = sc;
    for (j = 0; j < c->d; ++j) c->codes[r * c->d + j] = synth_e4m3_rne(x[j] / (double)sc);
  }
  free(x);
}

void synth_fp8_rows(uint64_t seed, uint64_t tid, uint64_t row_off, uint64_t rows, uint64_t d,
                    double scale, uint8_t *codes, float *scales) {
  fp8_ctx c = {synth_stream_base(seed, tid), row_off, d, scale, codes, scales};
  parallel_for(rows, 64, fp8_range, &c);
}

/* ---- int8 compact keys ------------------------------------------------------ */

static inline double bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

typedef struct { const uint16_t *k; uint64_t d, dc; const float *P; int8_t *c; float *cs; } compact_ctx;

static void compact_range(void *p, uint64_t lo, uint64_t hi) {
  compact_ctx *c = (compact_ctx *)p;
  double *y = (double *)malloc(sizeof(double) * c->dc);
  double *kv = (double *)malloc(sizeof(double) * c->d);
  for (uint64_t r = lo; r < hi; ++r) {
    for (uint64_t j = 0; j < c->d; ++j) kv[j] = bf16_value(c->k[r * c->d + j]);
    double amax = 0.0;
    for (uint64_t i = 0; i < c->dc; ++i) {
      double acc = 0.0;
      for (uint64_t j = 0; j < c->d; ++j) acc = fma((double)c->P[i * c->d + j], kv[j], acc);
      y[i] = acc;
      if (fabs(acc) > amax) amax = fabs(acc);
    }
    float sc = amax > 0.0 ? (float)(amax / 127.0) : 1.0f;
    c->cs[r] = sc;
    for (uint64_t i = 0; i < c->dc; ++i) {
      double t = rint(y[i] / (double)sc);
      if (t > 127.0) t = 127.0;
      if (t < -127.0) t = -127.0;
      c->c[r * c->dc + i] = (int8_t)t;
    }
  }
  free(y);
  free(kv);
}

void synth_compact_keys(const uint16_t *k_bf16, uint64_t rows, uint64_t d, const float *P, uint64_t dc,
                        int8_t *c, float *cs) {
  compact_ctx ctx = {k_bf16, d, dc, P, c, cs};
  parallel_for(rows, 256, compact_range, &ctx);
}

/* ---- product-quantisation codebooks and codes ------------------------------
 * The storage format of product-quantised indexer keys: each key's d dims split
 * into d / 4 pieces of 4, each piece stored as the one-byte index of an entry of
 * its piece's 256-entry codebook, the codebooks trained offline (k-means) and kept
 * as int8 entries with one fp32 scale for all of them.  Like the fp8 and int8
 * encoders above this only prepares input bytes: nothing here scores or selects. */

typedef struct { const uint16_t *k; uint64_t n, d, seed; int iters; double *cent; } pqtrain_ctx;

static void pqtrain_range(void *p, uint64_t lo, uint64_t hi) {
  pqtrain_ctx *c = (pqtrain_ctx *)p;
  uint64_t n = c->n, d = c->d;
  uint32_t *asg = (uint32_t *)malloc(sizeof(uint32_t) * (n ? n : 1));
  double *sum = (double *)malloc(sizeof(double) * 256 * 4);
  uint64_t *cnt = (uint64_t *)malloc(sizeof(uint64_t) * 256);
  for (uint64_t j = lo; j < hi; ++j) {
    double *cent = c->cent + j * 256 * 4;
    /* initial centroids: 256 sample points chosen by the seeded stream */
    uint64_t base = synth_stream_base(c->seed, 100 + j);
    for (int e = 0; e < 256; ++e) {
      uint64_t r = draw(base, (uint64_t)e) % n;
      for (int i = 0; i < 4; ++i) cent[e * 4 + i] = bf16_value(c->k[r * d + 4 * j + i]);
    }
    for (int it = 0; it < c->iters; ++it) {
      for (uint64_t x = 0; x < n; ++x) {
        double v[4];
        for (int i = 0; i < 4; ++i) v[i] = bf16_value(c->k[x * d + 4 * j + i]);
        double best = INFINITY;
        uint32_t bi = 0;
        for (uint32_t e = 0; e < 256; ++e) {
          double dd = 0.0;
          for (int i = 0; i < 4; ++i) {
            double t = v[i] - cent[e * 4 + i];
            dd += t * t;
          }
          if (dd < best) { best = dd; bi = e; }
        }
        asg[x] = bi;
      }
      memset(sum, 0, sizeof(double) * 256 * 4);
      memset(cnt, 0, sizeof(uint64_t) * 256);
      for (uint64_t x = 0; x < n; ++x) {
        cnt[asg[x]] += 1;
        for (int i = 0; i < 4; ++i) sum[asg[x] * 4 + i] += bf16_value(c->k[x * d + 4 * j + i]);
      }
      for (int e = 0; e < 256; ++e)
        if (cnt[e])
          for (int i = 0; i < 4; ++i) cent[e * 4 + i] = sum[e * 4 + i] / (double)cnt[e];
    }
  }
  free(asg); free(sum); free(cnt);
}

/* Codebooks from n bf16 keys [n, d]: `iters` Lloyd iterations per piece from 256
 * seeded sample points (an entry left empty keeps its place), then one scale
 * sigma = max |entry| / 127 and int8 entries rint(entry / sigma).
 * cb: [d / 4, 256, 4] int8. */
void synth_pq_codebook(const uint16_t *k, uint64_t n, uint64_t d, uint64_t seed, int iters, int8_t *cb,
                       float *sigma) {
  uint64_t np = d / 4;
  double *cent = (double *)malloc(sizeof(double) * np * 256 * 4);
  pqtrain_ctx c = {k, n, d, seed, iters, cent};
  parallel_for(np, 1, pqtrain_range, &c);
  double amax = 0.0;
  for (uint64_t i = 0; i < np * 256 * 4; ++i)
    if (fabs(cent[i]) > amax) amax = fabs(cent[i]);
  float sg = amax > 0.0 ? (float)(amax / 127.0) : 1.0f;
  for (uint64_t i = 0; i < np * 256 * 4; ++i) {
    double t = rint(cent[i] / (double)sg);
    if (t > 127.0) t = 127.0;
    if (t < -127.0) t = -127.0;
    cb[i] = (int8_t)t;
  }
  *sigma = sg;
  free(cent);
}

typedef struct { const uint16_t *k; uint64_t d; const int8_t *cb; double sigma; uint8_t *codes; } pqenc_ctx;

static void pqenc_range(void *p, uint64_t lo, uint64_t hi) {
  pqenc_ctx *c = (pqenc_ctx *)p;
  uint64_t d = c->d, np = d / 4;
  for (uint64_t r = lo; r < hi; ++r)
    for (uint64_t j = 0; j < np; ++j) {
      double v[4];
      for (int i = 0; i < 4; ++i) v[i] = bf16_value(c->k[r * d + 4 * j + i]);
      const int8_t *e0 = c->cb + j * 256 * 4;
      double best = INFINITY;
      int bi = 0;
      for (int e = 0; e < 256; ++e) {
        double dd = 0.0;
        for (int i = 0; i < 4; ++i) {
          double t = v[i] - c->sigma * (double)e0[e * 4 + i];
          dd += t * t;
        }
        if (dd < best) { best = dd; bi = e; }
      }
      c->codes[r * np + j] = (uint8_t)bi;
    }
}

/* Codes of bf16 keys [rows, d]: per piece the entry nearest (squared distance in
 * fp64, ties to the smaller index) among sigma * cb. codes: [rows, d / 4]. */
void synth_pq_encode(const uint16_t *k, uint64_t rows, uint64_t d, const int8_t *cb, float sigma, uint8_t *codes) {
  pqenc_ctx c = {k, d, cb, (double)sigma, codes};
  parallel_for(rows, 256, pqenc_range, &c);
}

int synth_threads(void) { return n_threads(); }
