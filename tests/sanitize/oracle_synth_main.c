/*
 * Sanitizer driver for the host C code of the test side: the seeded
 * generator (synth.c, included below as one translation unit) and the
 * float64 oracle (sps_oracle.c, compiled beside it). Built with
 * -fsanitize=address,undefined and no recovery, it walks every exported
 * routine over a small corpus with empty rows, ragged chunks and planted
 * CSR faults; any out-of-bounds access, leak or undefined operation ends
 * the run with a sanitizer report and a non-zero status.
 *
 * The arithmetic checks here are only consistency checks between routines
 * (a row of scores sums to the row sum the oracle reports); the oracle's
 * own pins live in the Python tests.
 */
#include "../../synth/synth.c"

#include <stdio.h>

int orc_validate_csr(int64_t n_rows, int64_t n_cols, int64_t nnz, const int32_t *indptr,
                     const int32_t *indices, const float *values, int64_t *first_bad_row);
void orc_row_norms(int64_t n_rows, const int32_t *indptr, const float *values, double *norm64,
                   float *inv32);
void orc_chunk_csc(int64_t dim, const int32_t *indptr, const int32_t *indices,
                   const float *values, const double *norm64, int64_t item_begin,
                   int64_t item_end, int32_t *col_ptr, int32_t *row, float *val);
void orc_set_thread_cpus(const int32_t *cpus, int n);
void orc_scores(const int32_t *q_indptr, const int32_t *q_indices, const float *q_values,
                const double *q_norm, const int32_t *i_indptr, const int32_t *i_indices,
                const float *i_values, const double *i_norm, const int64_t *q_rows,
                int64_t n_sel, int64_t item_begin, int64_t item_end, double *out,
                int n_threads);
void orc_chunk_row_sums(const int32_t *q_indptr, const int32_t *q_indices,
                        const float *q_values, const double *q_norm, int64_t n_q,
                        const int32_t *i_indptr, const int32_t *i_indices,
                        const float *i_values, const double *i_norm, int64_t n_items,
                        int64_t dim, int64_t chunk_size, double *row_sums, int n_threads,
                        int kind);
void orc_col_sums(const int32_t *q_indptr, const int32_t *q_indices, const float *q_values,
                  const double *q_norm, int64_t n_q, const int32_t *i_indptr,
                  const int32_t *i_indices, const float *i_values, const double *i_norm,
                  int64_t dim, int64_t item_begin, int64_t item_end, double *col_sums,
                  int kind);

#define CHECK(c)                                                              \
  do {                                                                        \
    if (!(c)) {                                                               \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);         \
      exit(2);                                                                \
    }                                                                         \
  } while (0)

typedef struct {
  int64_t n_rows, dim, nnz;
  int32_t *indptr, *indices;
  float *values;
} csr_t;

static csr_t make(const corpus_spec *sp, const uint8_t *force_empty) {
  csr_t m;
  m.n_rows = sp->n_rows;
  m.dim = sp->dim;
  int32_t *cnt = (int32_t *)malloc((size_t)m.n_rows * sizeof(int32_t));
  m.nnz = synth_row_nnz(sp, force_empty, cnt, 3);
  CHECK(m.nnz >= 0);
  m.indptr = (int32_t *)malloc((size_t)(m.n_rows + 1) * sizeof(int32_t));
  m.indptr[0] = 0;
  for (int64_t r = 0; r < m.n_rows; ++r) m.indptr[r + 1] = m.indptr[r] + cnt[r];
  free(cnt);
  /* one spare slot so that a zero-nnz matrix still has a valid pointer */
  m.indices = (int32_t *)malloc((size_t)(m.nnz + 1) * sizeof(int32_t));
  m.values = (float *)malloc((size_t)(m.nnz + 1) * sizeof(float));
  CHECK(synth_fill(sp, m.indptr, m.indices, m.values, 3) == 0);
  return m;
}

static void drop(csr_t *m) {
  free(m->indptr);
  free(m->indices);
  free(m->values);
}

static void run(int64_t n_items, int64_t n_q, int64_t dim, int64_t chunk, int idx_kind,
                int val_kind) {
  corpus_spec is = {n_items, dim, 77u, 0u, NNZ_POISSON, 9.0, 1.0, 1, 64, idx_kind, 1.1,
                    val_kind};
  corpus_spec qs = is;
  qs.n_rows = n_q;
  qs.matrix = 1u;
  uint8_t *empty_i = (uint8_t *)calloc((size_t)n_items, 1);
  uint8_t *empty_q = (uint8_t *)calloc((size_t)n_q, 1);
  for (int64_t r = 0; r < n_items; r += 13) empty_i[r] = 1;
  for (int64_t r = 1; r < n_q; r += 7) empty_q[r] = 1;
  csr_t I = make(&is, empty_i), Q = make(&qs, empty_q);
  free(empty_i);
  free(empty_q);

  int64_t bad = 7;
  CHECK(orc_validate_csr(I.n_rows, dim, I.nnz, I.indptr, I.indices, I.values, &bad) == 0);
  CHECK(bad == -1);
  CHECK(orc_validate_csr(Q.n_rows, dim, Q.nnz, Q.indptr, Q.indices, Q.values, &bad) == 0);

  double *in64 = (double *)malloc((size_t)n_items * sizeof(double));
  double *qn64 = (double *)malloc((size_t)n_q * sizeof(double));
  float *in32 = (float *)malloc((size_t)n_items * sizeof(float));
  orc_row_norms(n_items, I.indptr, I.values, in64, in32);
  orc_row_norms(n_q, Q.indptr, Q.values, qn64, NULL);
  CHECK(in64[0] == 0.0 && in32[0] == 0.0f);

  /* every chunk's inverted lists, the last one ragged */
  int32_t *col_ptr = (int32_t *)malloc((size_t)(dim + 1) * sizeof(int32_t));
  int32_t *row = (int32_t *)malloc((size_t)(I.nnz + 1) * sizeof(int32_t));
  float *val = (float *)malloc((size_t)(I.nnz + 1) * sizeof(float));
  for (int64_t b = 0; b < n_items; b += chunk) {
    int64_t e = b + chunk < n_items ? b + chunk : n_items;
    orc_chunk_csc(dim, I.indptr, I.indices, I.values, in64, b, e, col_ptr, row, val);
    CHECK(col_ptr[dim] == I.indptr[e] - I.indptr[b]);
  }

  /* all scores, unpinned threads, then pinned to cpu 0 */
  double *S = (double *)malloc((size_t)(n_q * n_items + 1) * sizeof(double));
  orc_scores(Q.indptr, Q.indices, Q.values, qn64, I.indptr, I.indices, I.values, in64, NULL,
             n_q, 0, n_items, S, 3);
  int32_t cpu0 = 0;
  orc_set_thread_cpus(&cpu0, 1);
  int64_t sel[3] = {n_q - 1, 0, n_q / 2};
  double *S3 = (double *)malloc((size_t)(3 * n_items + 1) * sizeof(double));
  orc_scores(Q.indptr, Q.indices, Q.values, qn64, I.indptr, I.indices, I.values, in64, sel, 3,
             0, n_items, S3, 2);
  orc_set_thread_cpus(NULL, 0);
  for (int s = 0; s < 3; ++s)
    for (int64_t i = 0; i < n_items; ++i) CHECK(S3[s * n_items + i] == S[sel[s] * n_items + i]);

  /* checksums of every kind */
  int64_t n_chunks = (n_items + chunk - 1) / chunk;
  double *rs = (double *)malloc((size_t)(n_chunks * n_q) * sizeof(double));
  double *cs = (double *)malloc((size_t)n_items * sizeof(double));
  for (int kind = 0; kind < 3; ++kind) {
    orc_chunk_row_sums(Q.indptr, Q.indices, Q.values, qn64, n_q, I.indptr, I.indices,
                       I.values, in64, n_items, dim, chunk, rs, 3, kind);
    orc_col_sums(Q.indptr, Q.indices, Q.values, qn64, n_q, I.indptr, I.indices, I.values,
                 in64, dim, 0, n_items, cs, kind);
    if (kind == 0) {
      for (int64_t q = 0; q < n_q; ++q) {
        double t = 0.0, u = 0.0;
        for (int64_t c = 0; c < n_chunks; ++c) t += rs[c * n_q + q];
        for (int64_t i = 0; i < n_items; ++i) u += S[q * n_items + i];
        CHECK(fabs(t - u) <= 1e-9 * (1.0 + fabs(u)));
      }
      for (int64_t i = 0; i < n_items; ++i) {
        double u = 0.0;
        for (int64_t q = 0; q < n_q; ++q) u += S[q * n_items + i];
        CHECK(fabs(cs[i] - u) <= 1e-9 * (1.0 + fabs(u)));
      }
    }
  }

  /* planted faults: each is reported with its row, and nothing is read
   * beyond the arrays */
  if (I.nnz >= 4) {
    int32_t keep = I.indices[1];
    int64_t r1 = 0;
    while (I.indptr[r1 + 1] < 2) ++r1;
    I.indices[1] = (int32_t)dim;
    CHECK(orc_validate_csr(I.n_rows, dim, I.nnz, I.indptr, I.indices, I.values, &bad) == 3);
    CHECK(bad == r1);
    I.indices[1] = keep;
    int32_t end = I.indptr[n_items];
    I.indptr[n_items] = end + 1;
    CHECK(orc_validate_csr(I.n_rows, dim, I.nnz, I.indptr, I.indices, I.values, &bad) == 1);
    I.indptr[n_items] = end;
  }

  free(S); free(S3); free(rs); free(cs); free(col_ptr); free(row); free(val);
  free(in64); free(qn64); free(in32);
  drop(&I);
  drop(&Q);
}

int main(void) {
  uint32_t ctr[4] = {1, 2, 3, 4}, key[2] = {5, 6}, out[4];
  synth_philox4x32_10(ctr, key, out);
  int64_t pick[40];
  CHECK(synth_subset(9u, 1u, 1000, 40, pick) == 0);
  run(1001, 23, 4000, 256, IDX_ZIPF, VAL_LOGNORMAL);
  run(300, 9, 70, 64, IDX_UNIFORM, VAL_NORMAL);          /* dense overlap, signed values */
  run(5, 3, 1000000, 2, IDX_UNIFORM, VAL_LOG1P_HALFNORMAL); /* wide, nearly empty */
  puts("oracle and generator: clean");
  return 0;
}
