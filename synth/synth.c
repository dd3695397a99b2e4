/*
 * synth.c -- seeded synthetic sparse-embedding corpora (CSR, fp32 values).
 *
 * This module only makes inputs. It holds none of the similarity
 * arithmetic: no norms, no dot products, no transposes. Both the float64
 * oracle and the GPU library are fed from it.
 *
 * Randomness: Philox4x32-10, the counter-based generator of Salmon, Moraes,
 * Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11).
 * Every (matrix, row, purpose) triple owns its own counter stream, so the
 * output does not depend on the number of threads.
 *
 * Workload shapes follow the page "稀疏嵌入批量相似度计算的工程化实践"
 * (Engineering practice of bulk similarity for sparse embeddings), §1
 * (50k queries x 2M items, dim 1.2M, mean nnz 43) and §3.2 (term ids
 * cluster in a dictionary prefix): heavy Zipf ranks sit at the lowest dims.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------- Philox4x32-10 ---------------- */

static void philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2],
                          uint32_t out[4]) {
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    uint32_t n1 = (uint32_t)p1;
    uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    uint32_t n3 = (uint32_t)p0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  philox4x32_10(ctr, key, out);
}

/* One stream: key = (seed, matrix), counter = (row lo, row hi, purpose, block). */
typedef struct {
  uint32_t key[2];
  uint32_t ctr[4];
  uint32_t buf[4];
  int pos;
} stream_t;

static void stream_init(stream_t *s, uint64_t seed, uint32_t matrix, uint64_t row,
                        uint32_t purpose) {
  s->key[0] = (uint32_t)seed;
  s->key[1] = (uint32_t)(seed >> 32) ^ (matrix * 0x85EBCA6Bu);
  s->ctr[0] = (uint32_t)row;
  s->ctr[1] = (uint32_t)(row >> 32);
  s->ctr[2] = purpose;
  s->ctr[3] = 0;
  s->pos = 4;
}

static uint32_t next_u32(stream_t *s) {
  if (s->pos == 4) {
    philox4x32_10(s->ctr, s->key, s->buf);
    s->ctr[3] += 1;
    s->pos = 0;
  }
  return s->buf[s->pos++];
}

/* uniform in the open interval (0, 1), 53 random bits */
static double next_unif(stream_t *s) {
  uint64_t hi = next_u32(s), lo = next_u32(s);
  uint64_t x = ((hi << 32) | lo) >> 11;
  return ((double)x + 0.5) * (1.0 / 9007199254740992.0);
}

/* uniform integer in [0, n) by rejection (no modulo bias) */
static uint64_t next_below(stream_t *s, uint64_t n) {
  if (n <= 1) return 0;
  if (n <= 0xFFFFFFFFull) {
    uint32_t lim = (uint32_t)(0x100000000ull - (0x100000000ull % n));
    for (;;) {
      uint32_t x = next_u32(s);
      if (lim == 0 || x < lim) return x % n;
    }
  }
  for (;;) {
    uint64_t x = ((uint64_t)next_u32(s) << 32) | next_u32(s);
    uint64_t lim = UINT64_MAX - (UINT64_MAX % n);
    if (x < lim) return x % n;
  }
}

/* standard normal, Box-Muller (one output per pair of uniforms) */
static double next_normal(stream_t *s) {
  double u1 = next_unif(s), u2 = next_unif(s);
  return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}

/* Poisson(lambda) by sequential inversion */
static int64_t next_poisson(stream_t *s, double lambda) {
  double u = next_unif(s);
  double p = exp(-lambda), F = p;
  int64_t k = 0;
  while (u > F && k < 100000) {
    k += 1;
    p *= lambda / (double)k;
    F += p;
    if (p == 0.0 && F < u) break;
  }
  return k;
}

/* ---------------- distributions of one corpus ---------------- */

enum { NNZ_UNIFORM = 0, NNZ_POISSON = 1, NNZ_LOGNORMAL = 2 };
enum { IDX_UNIFORM = 0, IDX_ZIPF = 1 };
enum { VAL_LOGNORMAL = 0, VAL_LOG1P_HALFNORMAL = 1, VAL_NORMAL = 2 };

typedef struct {
  int64_t n_rows, dim;
  uint64_t seed;
  uint32_t matrix;          /* 0 = items, 1 = queries, other = free use */
  int nnz_kind;             /* NNZ_* */
  double nnz_a, nnz_b;      /* uniform: [a,b]; poisson: lambda=a, min=b; lognormal: mu=a, sigma=b */
  int64_t nnz_min, nnz_max; /* clip */
  int idx_kind;             /* IDX_* */
  double zipf_s;
  int val_kind;             /* VAL_* */
} corpus_spec;

typedef struct {
  const corpus_spec *sp;
  const double *cdf;       /* zipf cdf over ranks 1..dim, cdf[dim-1] == 1 */
  const int64_t *guide;    /* guide table of size n_guide+1 */
  int64_t n_guide;
} sampler_t;

static int64_t sample_zipf(const sampler_t *sm, stream_t *s) {
  double u = next_unif(s);
  int64_t g = (int64_t)(u * (double)sm->n_guide);
  if (g >= sm->n_guide) g = sm->n_guide - 1;
  int64_t i = sm->guide[g];
  const int64_t last = sm->sp->dim - 1;
  while (i < last && sm->cdf[i] <= u) ++i;
  return i; /* rank i+1 -> dim i */
}

static int64_t draw_nnz(const corpus_spec *sp, int64_t row) {
  stream_t s;
  stream_init(&s, sp->seed, sp->matrix, (uint64_t)row, 0);
  int64_t k = 0;
  if (sp->nnz_kind == NNZ_UNIFORM) {
    int64_t a = (int64_t)sp->nnz_a, b = (int64_t)sp->nnz_b;
    k = a + (int64_t)next_below(&s, (uint64_t)(b - a + 1));
  } else if (sp->nnz_kind == NNZ_POISSON) {
    k = next_poisson(&s, sp->nnz_a);
  } else {
    double z = next_normal(&s);
    k = (int64_t)rint(exp(sp->nnz_a + sp->nnz_b * z));
  }
  if (k < sp->nnz_min) k = sp->nnz_min;
  if (k > sp->nnz_max) k = sp->nnz_max;
  if (k > sp->dim) k = sp->dim;
  return k;
}

static int cmp_i32(const void *a, const void *b) {
  int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
  return (x > y) - (x < y);
}

/* open-addressing set of dims, reused across rows of one thread */
typedef struct {
  int32_t *slot;
  int64_t cap; /* power of two */
} dimset_t;

static void dimset_reset(dimset_t *h, int64_t need) {
  int64_t cap = 64;
  while (cap < 4 * need) cap <<= 1;
  if (cap > h->cap) {
    free(h->slot);
    h->slot = (int32_t *)malloc((size_t)cap * sizeof(int32_t));
    h->cap = cap;
  }
  memset(h->slot, 0xFF, (size_t)h->cap * sizeof(int32_t));
}

/* returns 1 if inserted, 0 if already present */
static int dimset_insert(dimset_t *h, int32_t d) {
  uint64_t m = (uint64_t)h->cap - 1;
  uint64_t i = ((uint64_t)(uint32_t)d * 0x9E3779B97F4A7C15ull) >> 17;
  for (;;) {
    i &= m;
    if (h->slot[i] == d) return 0;
    if (h->slot[i] < 0) { h->slot[i] = d; return 1; }
    ++i;
  }
}

static void fill_row(const sampler_t *sm, dimset_t *hs, int64_t row, int64_t k,
                     int32_t *idx, float *val) {
  const corpus_spec *sp = sm->sp;
  if (k == 0) return;
  stream_t si;
  stream_init(&si, sp->seed, sp->matrix, (uint64_t)row, 1);
  dimset_reset(hs, k);
  int64_t got = 0;
  /* successive draws; repeats are rejected, so the row keeps the first k
   * distinct dims in draw order (sampling without replacement) */
  while (got < k) {
    int64_t d = (sp->idx_kind == IDX_ZIPF) ? sample_zipf(sm, &si)
                                           : (int64_t)next_below(&si, (uint64_t)sp->dim);
    if (dimset_insert(hs, (int32_t)d)) idx[got++] = (int32_t)d;
  }
  qsort(idx, (size_t)k, sizeof(int32_t), cmp_i32);
  stream_t sv;
  stream_init(&sv, sp->seed, sp->matrix, (uint64_t)row, 2);
  for (int64_t j = 0; j < k; ++j) {
    double v;
    if (sp->val_kind == VAL_LOGNORMAL) {
      v = exp(next_normal(&sv));
    } else if (sp->val_kind == VAL_LOG1P_HALFNORMAL) {
      double z;
      do { z = fabs(next_normal(&sv)); } while (!(z > 0.0));
      v = log1p(z);
    } else {
      v = next_normal(&sv);
    }
    val[j] = (float)v;
    if (sp->val_kind != VAL_NORMAL && !(val[j] > 0.0f)) val[j] = 1.17549435e-38f;
  }
}

/* ---------------- threaded drivers ---------------- */

typedef struct {
  const corpus_spec *sp;
  const sampler_t *sm;
  int64_t r0, r1;
  int32_t *nnz_out;          /* pass 1 */
  const int32_t *indptr;     /* pass 2 */
  int32_t *indices;
  float *values;
  const uint8_t *force_empty;
} work_t;

static void *pass1(void *arg) {
  work_t *w = (work_t *)arg;
  for (int64_t r = w->r0; r < w->r1; ++r) {
    int64_t k = draw_nnz(w->sp, r);
    if (w->force_empty && w->force_empty[r]) k = 0;
    w->nnz_out[r] = (int32_t)k;
  }
  return NULL;
}

static void *pass2(void *arg) {
  work_t *w = (work_t *)arg;
  dimset_t hs = {NULL, 0};
  for (int64_t r = w->r0; r < w->r1; ++r) {
    int64_t b = w->indptr[r], e = w->indptr[r + 1];
    fill_row(w->sm, &hs, r, e - b, w->indices + b, w->values + b);
  }
  free(hs.slot);
  return NULL;
}

static void run_threads(void *(*fn)(void *), work_t *proto, int64_t n_rows, int n_threads) {
  if (n_threads < 1) n_threads = 1;
  if (n_threads > 256) n_threads = 256;
  pthread_t th[256];
  work_t w[256];
  int64_t per = (n_rows + n_threads - 1) / n_threads;
  int launched = 0;
  for (int t = 0; t < n_threads; ++t) {
    w[t] = *proto;
    w[t].r0 = (int64_t)t * per;
    w[t].r1 = w[t].r0 + per < n_rows ? w[t].r0 + per : n_rows;
    if (w[t].r0 >= w[t].r1) break;
    if (pthread_create(&th[t], NULL, fn, &w[t]) != 0) { fn(&w[t]); th[t] = 0; }
    launched = t + 1;
  }
  for (int t = 0; t < launched; ++t)
    if (th[t]) pthread_join(th[t], NULL);
}

/*
 * Pass 1: per-row nnz into nnz_out[n_rows]. force_empty (nullable) marks
 * rows forced to nnz 0. Returns the total nnz, or -1 if it exceeds 2^31-1.
 */
int64_t synth_row_nnz(const corpus_spec *sp, const uint8_t *force_empty, int32_t *nnz_out,
                      int n_threads) {
  work_t proto;
  memset(&proto, 0, sizeof proto);
  proto.sp = sp;
  proto.nnz_out = nnz_out;
  proto.force_empty = force_empty;
  run_threads(pass1, &proto, sp->n_rows, n_threads);
  int64_t tot = 0;
  for (int64_t r = 0; r < sp->n_rows; ++r) tot += nnz_out[r];
  return tot > 2147483647ll ? -1 : tot;
}

/* Pass 2: indices/values for a CSR whose indptr was built from pass 1. */
int synth_fill(const corpus_spec *sp, const int32_t *indptr, int32_t *indices, float *values,
               int n_threads) {
  double *cdf = NULL;
  int64_t *guide = NULL;
  sampler_t sm;
  memset(&sm, 0, sizeof sm);
  sm.sp = sp;
  if (sp->idx_kind == IDX_ZIPF) {
    int64_t D = sp->dim;
    cdf = (double *)malloc((size_t)D * sizeof(double));
    if (!cdf) return -1;
    double acc = 0.0;
    for (int64_t r = 0; r < D; ++r) {
      acc += pow((double)(r + 1), -sp->zipf_s);
      cdf[r] = acc;
    }
    for (int64_t r = 0; r < D; ++r) cdf[r] /= acc;
    cdf[D - 1] = 1.0;
    int64_t G = D;
    guide = (int64_t *)malloc((size_t)(G + 1) * sizeof(int64_t));
    if (!guide) { free(cdf); return -1; }
    int64_t i = 0;
    for (int64_t g = 0; g <= G; ++g) {
      double t = (double)g / (double)G;
      while (i < D - 1 && cdf[i] <= t) ++i;
      guide[g] = i;
    }
    sm.cdf = cdf;
    sm.guide = guide;
    sm.n_guide = G;
  }
  work_t proto;
  memset(&proto, 0, sizeof proto);
  proto.sp = sp;
  proto.sm = &sm;
  proto.indptr = indptr;
  proto.indices = indices;
  proto.values = values;
  run_threads(pass2, &proto, sp->n_rows, n_threads);
  free(cdf);
  free(guide);
  return 0;
}

/* First k entries of a seeded Fisher-Yates shuffle of 0..n-1 (distinct). */
int synth_subset(uint64_t seed, uint32_t matrix, int64_t n, int64_t k, int64_t *out) {
  if (k > n || k < 0) return -1;
  int64_t *perm = (int64_t *)malloc((size_t)n * sizeof(int64_t));
  if (!perm) return -1;
  for (int64_t i = 0; i < n; ++i) perm[i] = i;
  stream_t s;
  stream_init(&s, seed, matrix, 0, 3);
  for (int64_t i = 0; i < k; ++i) {
    int64_t j = i + (int64_t)next_below(&s, (uint64_t)(n - i));
    int64_t t = perm[i]; perm[i] = perm[j]; perm[j] = t;
    out[i] = perm[i];
  }
  free(perm);
  return 0;
}
