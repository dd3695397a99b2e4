/*
 * sps_oracle.c -- plain float64 CPU oracle for exact all-pairs sparse cosine.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library. It shares no code with the GPU
 * library: no headers, helpers, tables or kernels.
 *
 * Source of every formula: the page "稀疏嵌入批量相似度计算的工程化实践"
 * (Engineering practice of bulk similarity for sparse embeddings).
 *   - cosine = dot / (||u||_2 ||v||_2)                        §3.1, first equation
 *   - dot over the shared support only                        §3.1, second equation
 *   - two sorted index arrays, two pointers, multiply-add
 *     only on equal indices, strictly ordered indices needed   §3.1 (two-pointer merge, note)
 *   - row norm from the stored nonzeros only                  §5.2, detail one
 *   - items processed in contiguous chunks, chunk indptr
 *     rebased to the chunk's first entry                      §4.4 (bulk_similarity loop)
 *   - output: full (n_query, n_item) matrix of normalised
 *     cosines, error below 1e-6                               §2.3
 *   - division by the two norms after the dot                 §4.4 (normalise after compute)
 *
 * Readings where the page is silent (also listed in the design notes):
 *   - a row whose norm is 0 (empty, or only stored zeros) scores 0 against
 *     everything, itself included;
 *   - the reference inverted list of a chunk is the textbook stable counting
 *     sort: col_ptr over all dims, chunk-local item ids ascending within each
 *     dim, values v / ||item|| rounded once to float32;
 *   - fp32 inverse norms are fl32(1 / ||row||), rounded once from float64.
 *
 * Compile-time ORC_MUTANT=k plants one deliberate mistake; the test suite
 * builds those variants to show its pins catch each one. The default build
 * (ORC_MUTANT undefined or 0) is the oracle.
 */
#define _GNU_SOURCE /* pthread_setaffinity_np */
#include <math.h>
#include <pthread.h>
#include <sched.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef ORC_MUTANT
#define ORC_MUTANT 0
#endif

/* ------------------------------------------------------------------ */
/* CSR validation (§3.1 note: the merge needs strictly ordered indices) */
/* ------------------------------------------------------------------ */

/* 0 ok; 1 bad indptr; 2 indices not strictly ascending within a row;
 * 3 index outside [0, n_cols); 4 non-finite value. */
int orc_validate_csr(int64_t n_rows, int64_t n_cols, int64_t nnz, const int32_t *indptr,
                     const int32_t *indices, const float *values, int64_t *first_bad_row) {
  *first_bad_row = -1;
  if (indptr[0] != 0 || (int64_t)indptr[n_rows] != nnz) {
    *first_bad_row = 0;
    return 1;
  }
  for (int64_t r = 0; r < n_rows; ++r) {
    int64_t b = indptr[r], e = indptr[r + 1];
    if (e < b || e > nnz) { *first_bad_row = r; return 1; }
    for (int64_t k = b; k < e; ++k) {
      if (indices[k] < 0 || (int64_t)indices[k] >= n_cols) { *first_bad_row = r; return 3; }
      if (k > b && indices[k] <= indices[k - 1]) { *first_bad_row = r; return 2; }
      if (!isfinite(values[k])) { *first_bad_row = r; return 4; }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------ */
/* Row norms (§5.2: square the stored nonzeros, sum, square root)      */
/* ------------------------------------------------------------------ */

void orc_row_norms(int64_t n_rows, const int32_t *indptr, const float *values, double *norm64,
                   float *inv32) {
  for (int64_t r = 0; r < n_rows; ++r) {
    double s = 0.0;
    for (int64_t k = indptr[r]; k < indptr[r + 1]; ++k) {
      double v = (double)values[k];
#if ORC_MUTANT == 2
      s += fabs(v);
#else
      s += v * v;
#endif
    }
    double n = sqrt(s);
    norm64[r] = n;
    if (inv32) inv32[r] = (n > 0.0) ? (float)(1.0 / n) : 0.0f;
  }
}

/* ------------------------------------------------------------------ */
/* Reference inverted lists of one item chunk [item_begin, item_end)   */
/* (chunk slicing as in §4.4; transpose by stable counting sort)       */
/* ------------------------------------------------------------------ */

void orc_chunk_csc(int64_t dim, const int32_t *indptr, const int32_t *indices,
                   const float *values, const double *norm64, int64_t item_begin,
                   int64_t item_end, int32_t *col_ptr, int32_t *row, float *val) {
  const int64_t base = indptr[item_begin];
  const int64_t cnnz = (int64_t)indptr[item_end] - base;
  int32_t *cursor = (int32_t *)calloc((size_t)dim, sizeof(int32_t));
  /* counts */
  memset(col_ptr, 0, (size_t)(dim + 1) * sizeof(int32_t));
  for (int64_t k = base; k < base + cnnz; ++k) col_ptr[indices[k] + 1] += 1;
  /* exclusive prefix: col_ptr[d] = entries with dim < d */
  for (int64_t d = 0; d < dim; ++d) col_ptr[d + 1] += col_ptr[d];
  for (int64_t d = 0; d < dim; ++d) cursor[d] = col_ptr[d];
  /* stable scatter in item order */
#if ORC_MUTANT == 5
  for (int64_t i = item_end - 1; i >= item_begin; --i) {
#else
  for (int64_t i = item_begin; i < item_end; ++i) {
#endif
    const double n = norm64[i];
    for (int64_t k = indptr[i]; k < indptr[i + 1]; ++k) {
      const int32_t d = indices[k];
      const int32_t p = cursor[d]++;
#if ORC_MUTANT == 6
      row[p] = (int32_t)i;
#else
      row[p] = (int32_t)(i - item_begin);
#endif
      val[p] = (n > 0.0) ? (float)((double)values[k] / n) : 0.0f;
    }
  }
  free(cursor);
}

/* ------------------------------------------------------------------ */
/* Scores by per-pair two-pointer merge (§3.1), division after (§4.4)  */
/* ------------------------------------------------------------------ */

static double pair_dot(const int32_t *qi, const float *qv, int64_t qn, const int32_t *ii,
                       const float *iv, int64_t in) {
  double dot = 0.0;
  int64_t a = 0, b = 0;
  while (a < qn && b < in) {
    const int32_t x = qi[a], y = ii[b];
    if (x < y) {
#if ORC_MUTANT == 1
      ++b;
#else
      ++a;
#endif
    } else if (x > y) {
      ++b;
    } else {
#if ORC_MUTANT == 8
      dot += (double)qv[a] * (double)qv[a];
#else
      dot += (double)qv[a] * (double)iv[b];
#endif
      ++a;
      ++b;
    }
  }
  return dot;
}

static double cosine_from(double dot, double nq, double ni) {
#if ORC_MUTANT == 3
  return dot / (nq * ni);
#elif ORC_MUTANT == 4
  return (nq > 0.0 && ni > 0.0) ? dot / nq : 0.0;
#else
  return (nq > 0.0 && ni > 0.0) ? dot / (nq * ni) : 0.0;
#endif
}

typedef struct {
  const int32_t *q_indptr, *q_indices; const float *q_values; const double *q_norm;
  const int32_t *i_indptr, *i_indices; const float *i_values; const double *i_norm;
  const int64_t *q_rows; int64_t n_sel;
  int64_t item_begin, item_end;
  double *out;
  int64_t next; /* shared row counter */
  pthread_mutex_t mu;
} score_job;

static void *score_worker(void *arg) {
  score_job *J = (score_job *)arg;
  const int64_t width = J->item_end - J->item_begin;
  for (;;) {
    pthread_mutex_lock(&J->mu);
    int64_t s = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (s >= J->n_sel) break;
    const int64_t q = J->q_rows ? J->q_rows[s] : s;
    const int64_t qb = J->q_indptr[q], qe = J->q_indptr[q + 1];
    double *o = J->out + s * width;
    for (int64_t i = J->item_begin; i < J->item_end; ++i) {
      const int64_t ib = J->i_indptr[i], ie = J->i_indptr[i + 1];
      double dot = pair_dot(J->q_indices + qb, J->q_values + qb, qe - qb, J->i_indices + ib,
                            J->i_values + ib, ie - ib);
      o[i - J->item_begin] = cosine_from(dot, J->q_norm[q], J->i_norm[i]);
    }
  }
  return NULL;
}

/* Optional thread placement for orc_scores (timing runs): thread t (the
 * caller is thread 0) runs on cpus[t % n]; n = 0 leaves placement to the OS.
 * Placement only; it changes nothing in the arithmetic. */
static int g_pin_n = 0;
static int g_pin_cpus[256];

void orc_set_thread_cpus(const int32_t *cpus, int n) {
  if (n < 0) n = 0;
  if (n > 256) n = 256;
  for (int k = 0; k < n; ++k) g_pin_cpus[k] = cpus[k];
  g_pin_n = n;
}

static void pin_self(int t) {
  if (g_pin_n <= 0) return;
  cpu_set_t set;
  CPU_ZERO(&set);
  CPU_SET(g_pin_cpus[t % g_pin_n], &set);
  pthread_setaffinity_np(pthread_self(), sizeof set, &set);
}

typedef struct {
  void *job;
  int t;
} pinned_arg;

static void *score_worker(void *arg);

static void *pinned_score_worker(void *arg) {
  pinned_arg *p = (pinned_arg *)arg;
  pin_self(p->t);
  return score_worker(p->job);
}

/* out[s * (item_end-item_begin) + (i-item_begin)] = S[q_rows[s], i] (q_rows NULL: s) */
void orc_scores(const int32_t *q_indptr, const int32_t *q_indices, const float *q_values,
                const double *q_norm, const int32_t *i_indptr, const int32_t *i_indices,
                const float *i_values, const double *i_norm, const int64_t *q_rows,
                int64_t n_sel, int64_t item_begin, int64_t item_end, double *out,
                int n_threads) {
  score_job J;
  J.q_indptr = q_indptr; J.q_indices = q_indices; J.q_values = q_values; J.q_norm = q_norm;
  J.i_indptr = i_indptr; J.i_indices = i_indices; J.i_values = i_values; J.i_norm = i_norm;
  J.q_rows = q_rows; J.n_sel = n_sel; J.item_begin = item_begin; J.item_end = item_end;
  J.out = out; J.next = 0;
  pthread_mutex_init(&J.mu, NULL);
  if (n_threads < 1) n_threads = 1;
  if (n_threads > 256) n_threads = 256;
  pthread_t th[256];
  pinned_arg pa[256];
  int started = 0;
  for (int t = 1; t < n_threads; ++t) {
    pa[t].job = &J;
    pa[t].t = t;
    if (pthread_create(&th[started], NULL, pinned_score_worker, &pa[t]) == 0) ++started;
  }
  /* the calling thread works too, on cpus[0] when pinned, then gets its placement back */
  cpu_set_t before;
  const int restore = g_pin_n > 0 &&
                      pthread_getaffinity_np(pthread_self(), sizeof before, &before) == 0;
  pin_self(0);
  score_worker(&J);
  if (restore) pthread_setaffinity_np(pthread_self(), sizeof before, &before);
  for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
  pthread_mutex_destroy(&J.mu);
}

/* ------------------------------------------------------------------ */
/* Closed-form chunk checksums (linearity of the dot product)          */
/*   sum_{i in chunk} S[q,i] = q^ . (sum_{i in chunk} i^)               */
/*   sum_q S[q,i]            = (sum_q q^) . i^                          */
/* where x^ = x / ||x|| (0 for a zero-norm row).                        */
/*                                                                    */
/* The same closed forms hold with every normalised value x passed    */
/* through t() on both sides, since the sums are over products of     */
/* matched entries: kind 0 t(x) = x (the sums of S); kind 1 t(x) = |x| */
/* (the sums of sum_d |q^_d i^_d|, the scale of a pair's rounding      */
/* error); kind 2 t(x) = 1 for every stored entry of a row with a      */
/* non-zero norm (the number of shared dims, summed over the pairs).   */
/* ------------------------------------------------------------------ */

static double orc_t(double x, int kind) {
#if ORC_MUTANT == 9
  if (kind == 1) return x;
#else
  if (kind == 1) return fabs(x);
#endif
  if (kind == 2) return 1.0;
  return x;
}

typedef struct {
  const int32_t *q_indptr, *q_indices; const float *q_values; const double *q_norm;
  int64_t n_q;
  const int32_t *i_indptr, *i_indices; const float *i_values; const double *i_norm;
  int64_t n_items, dim, chunk_size, n_chunks;
  double *row_sums; /* n_chunks x n_q */
  int kind;
  int64_t next;
  pthread_mutex_t mu;
} rowsum_job;

static void *rowsum_worker(void *arg) {
  rowsum_job *J = (rowsum_job *)arg;
  double *s = (double *)calloc((size_t)J->dim, sizeof(double));
  for (;;) {
    pthread_mutex_lock(&J->mu);
    int64_t c = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (c >= J->n_chunks) break;
    const int64_t b = c * J->chunk_size;
    const int64_t e = (b + J->chunk_size < J->n_items) ? b + J->chunk_size : J->n_items;
    for (int64_t i = b; i < e; ++i) {
      const double n = J->i_norm[i];
      if (!(n > 0.0)) continue;
      for (int64_t k = J->i_indptr[i]; k < J->i_indptr[i + 1]; ++k)
        s[J->i_indices[k]] += orc_t((double)J->i_values[k] / n, J->kind);
    }
    double *out = J->row_sums + c * J->n_q;
    for (int64_t q = 0; q < J->n_q; ++q) {
      const double n = J->q_norm[q];
      double acc = 0.0;
      if (n > 0.0) {
        for (int64_t k = J->q_indptr[q]; k < J->q_indptr[q + 1]; ++k) {
#if ORC_MUTANT == 7
          acc += orc_t((double)J->q_values[k], J->kind) * s[J->q_indices[k]];
#else
          acc += orc_t((double)J->q_values[k] / n, J->kind) * s[J->q_indices[k]];
#endif
        }
      }
      out[q] = acc;
    }
    /* clear only what was touched */
    for (int64_t i = b; i < e; ++i)
      for (int64_t k = J->i_indptr[i]; k < J->i_indptr[i + 1]; ++k) s[J->i_indices[k]] = 0.0;
  }
  free(s);
  return NULL;
}

/* row_sums[c * n_q + q] = sum over items of chunk c of S[q, i], for every
 * chunk (kind 0; kinds 1 and 2 as above) */
void orc_chunk_row_sums(const int32_t *q_indptr, const int32_t *q_indices,
                        const float *q_values, const double *q_norm, int64_t n_q,
                        const int32_t *i_indptr, const int32_t *i_indices,
                        const float *i_values, const double *i_norm, int64_t n_items,
                        int64_t dim, int64_t chunk_size, double *row_sums, int n_threads,
                        int kind) {
  rowsum_job J;
  J.kind = kind;
  J.q_indptr = q_indptr; J.q_indices = q_indices; J.q_values = q_values; J.q_norm = q_norm;
  J.n_q = n_q;
  J.i_indptr = i_indptr; J.i_indices = i_indices; J.i_values = i_values; J.i_norm = i_norm;
  J.n_items = n_items; J.dim = dim; J.chunk_size = chunk_size;
  J.n_chunks = (n_items + chunk_size - 1) / chunk_size;
  J.row_sums = row_sums; J.next = 0;
  pthread_mutex_init(&J.mu, NULL);
  if (n_threads < 1) n_threads = 1;
  if (n_threads > 256) n_threads = 256;
  pthread_t th[256];
  int started = 0;
  for (int t = 1; t < n_threads; ++t)
    if (pthread_create(&th[started], NULL, rowsum_worker, &J) == 0) ++started;
  rowsum_worker(&J);
  for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
  pthread_mutex_destroy(&J.mu);
}

/* col_sums[i - item_begin] = sum over all queries of S[q, i] (kind 0; kinds
 * 1 and 2 as above) */
void orc_col_sums(const int32_t *q_indptr, const int32_t *q_indices, const float *q_values,
                  const double *q_norm, int64_t n_q, const int32_t *i_indptr,
                  const int32_t *i_indices, const float *i_values, const double *i_norm,
                  int64_t dim, int64_t item_begin, int64_t item_end, double *col_sums,
                  int kind) {
  double *qbar = (double *)calloc((size_t)dim, sizeof(double));
  for (int64_t q = 0; q < n_q; ++q) {
    const double n = q_norm[q];
    if (!(n > 0.0)) continue;
    for (int64_t k = q_indptr[q]; k < q_indptr[q + 1]; ++k)
      qbar[q_indices[k]] += orc_t((double)q_values[k] / n, kind);
  }
  for (int64_t i = item_begin; i < item_end; ++i) {
    const double n = i_norm[i];
    double acc = 0.0;
    if (n > 0.0)
      for (int64_t k = i_indptr[i]; k < i_indptr[i + 1]; ++k)
        acc += qbar[i_indices[k]] * orc_t((double)i_values[k] / n, kind);
    col_sums[i - item_begin] = acc;
  }
  free(qbar);
}
