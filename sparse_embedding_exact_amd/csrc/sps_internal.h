// sps_internal.h -- launchers shared by the C-ABI layer and the kernel file.
// Not part of the public interface (include/sps.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sps {

// flags block (device, 16 int32): [0] structural fault bits (1 indptr,
// 4 index range), [1] other fault bits (2 order/duplicate, 8 non-finite),
// [2..3] uint64 min key (row << 3 | reason) of the first faulty row.
constexpr int kFlagsInts = 16;

hipError_t launch_fill_i32(int32_t *p, int64_t n, int32_t v, hipStream_t s);
hipError_t launch_csr_check(int64_t n_rows, int64_t n_cols, int64_t nnz, const int32_t *indptr,
                            const int32_t *indices, const float *values, int full,
                            int32_t *flags, hipStream_t s);
hipError_t launch_row_norms(int64_t n_rows, int64_t nnz, const int32_t *indptr,
                            const float *values, const int32_t *flags, float *inv32,
                            double *norm64, hipStream_t s);

// ---- items: per-chunk inverted lists ----
struct ItemsDev {
  int64_t n_items, dim, nnz;
  int32_t chunk_size, num_chunks;
  const int32_t *indptr, *indices;
  const float *values;
  float *inv_norm;      // persistent
  int32_t *col_ptr;     // persistent, num_chunks * (dim+1)
  uint16_t *row;        // persistent, nnz
  float *val;           // persistent, nnz
  int32_t *chunk_base;  // persistent, num_chunks + 1
  int32_t *flags;       // scratch
  double *norm64;       // scratch
  int32_t *ticket;      // scratch
  uint16_t *trow;       // scratch
  float *tval;          // scratch
  int32_t *mlist;       // scratch, nnz/2 + num_chunks + 1
  int32_t *mcount;      // scratch, num_chunks
};
hipError_t launch_prepare_items(const ItemsDev &d, hipStream_t s);

// ---- queries: row groups ----
struct QueriesDev {
  int64_t n_rows, dim, nnz;
  int32_t R, n_groups;
  const int32_t *indptr, *indices;
  const float *values;
  int32_t *flags;
  float *inv_norm;
  double *norm64;     // n_rows
  int32_t *grp_ptr;   // n_groups + 1
  int32_t *grp_dim;   // nnz
  float *grp_val;     // nnz * R: fl32(q / |q|) * 2^30 per row (0 where absent)
};
hipError_t launch_prepare_queries(const QueriesDev &d, hipStream_t s);

// ---- scoring ----
struct ScoreArgs {
  const int32_t *grp_ptr, *grp_dim;
  const float *grp_val, *q_inv;
  int64_t n_q, dim;
  int32_t R, n_groups;
  const int32_t *col_ptr;     // the chunk's col_ptr (dim+1), chunk-relative offsets
  const uint16_t *row;        // all chunks' item ids; the chunk starts at chunk_base[chunk]
  const float *val;
  const int32_t *chunk_base;  // device, num_chunks + 1
  int32_t chunk, chunk_len;
  float *out;
  int64_t ld;
  double *row_sums;
};
// Largest R (rows per workgroup) supported for a chunk length, given the
// device's LDS per workgroup; 0 if none fits.
int score_max_rows(int32_t chunk_len, size_t lds_limit);
size_t score_lds_bytes(int R, int32_t chunk_len);
hipError_t launch_score(const ScoreArgs &a, hipStream_t s);

}  // namespace sps
