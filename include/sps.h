/*
 * sps.h -- exact all-pairs cosine similarity of sparse embeddings on MI355X
 * (gfx950), C ABI.
 *
 * What it computes. The page "稀疏嵌入批量相似度计算的工程化实践"
 * (Engineering practice of bulk similarity for sparse embeddings) defines
 * the result: for CSR query rows q and CSR item rows i over the same
 * dimension,
 *
 *     S[q, i] = (sum over d in supp q ∩ supp i of q_d * i_d) / (|q|_2 |i|_2)
 *
 * (§3.1, both equations), a full (n_query, n_item) float32 matrix with no
 * top-K and no approximation (§2.3), produced item chunk by item chunk
 * (8192 items per chunk in §2.2 and §4.4). A row whose norm is 0 scores 0
 * against every row (the page is silent; this library's convention).
 *
 * How. Items are prepared once: their L2 norms (§5.2, from the stored
 * nonzeros only) and, for every slice of a chunk, inverted lists (a CSC,
 * values pre-divided by the item norm). Queries are prepared once per batch.
 * Each chunk is then scored by one kernel launch that accumulates query
 * nonzero x posting-list products in on-chip (LDS) accumulators and writes
 * full output rows.
 *
 * Conventions for every call:
 *  - Pointers marked DEVICE are device (HBM) addresses; the caller owns
 *    every device buffer (inputs, workspaces, outputs) and keeps it alive
 *    until the stream work that uses it has completed.
 *  - `stream` is a hipStream_t (NULL = the default stream). Calls that take
 *    a stream only enqueue work and return; they never synchronise unless
 *    documented. Enqueued work runs in stream order.
 *  - Every call returns an sps_status; nothing aborts, throws or exits.
 *    On an error no work has been enqueued, and sps_last_error_message()
 *    (thread-local) holds a detail string.
 *  - Sizes are 64-bit on the interface; row counts, nnz and dims must be
 *    below 2^31, and the item nnz below 2^29 - 64 (postings are addressed
 *    with 32-bit byte offsets) (SPS_ERR_OVERFLOW otherwise).
 *  - Input CSR must be canonical: indptr[0] = 0, non-decreasing,
 *    indptr[n_rows] = nnz, column indices strictly ascending within a row
 *    and inside [0, n_cols), values finite (§3.1 note: the merge needs
 *    strictly ordered indices). The prepare calls check the structure on
 *    the device: on a structural fault (indptr out of order or range, an
 *    index outside [0, n_cols)) they do no out-of-range access, still
 *    return SPS_OK, and the handle scores every row of that corpus or batch
 *    as 0. They report nothing to the host: callers with untrusted input
 *    run sps_validate_csr first (synchronous; it names the first faulty row
 *    and the reason).
 */
#ifndef SPS_H
#define SPS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. The type is a plain 32-bit integer, so any value a caller
 * hands back (sps_status_string(-99), say) is well defined on both sides. */
typedef int32_t sps_status;
enum {
  SPS_OK = 0,
  SPS_ERR_INVALID_ARGUMENT = -1,   /* NULL pointer, negative size, bad chunk size, ... */
  SPS_ERR_BAD_CSR = -2,            /* sps_validate_csr found a non-canonical CSR */
  SPS_ERR_DIM_MISMATCH = -3,       /* queries and items have different n_cols */
  SPS_ERR_WORKSPACE_TOO_SMALL = -4,/* a workspace is smaller than its sizing call said */
  SPS_ERR_CHUNK_RANGE = -5,        /* chunk index outside [0, num_chunks) */
  SPS_ERR_OVERFLOW = -6,           /* a size reaches 2^31 (or a byte count overflows) */
  SPS_ERR_HIP = -7,                /* a HIP runtime call or launch failed */
  SPS_ERR_UNSUPPORTED = -8         /* e.g. chunk too large for the device's LDS */
};

/* A CSR matrix. n_rows, n_cols and nnz are host values; the three arrays
 * are DEVICE arrays: indptr[n_rows+1] int32, indices[nnz] int32,
 * values[nnz] float32 (§4.2 and §3.2 of the page use int32 indptr). */
typedef struct {
  int64_t n_rows;
  int64_t n_cols;
  int64_t nnz;
  const int32_t *indptr;
  const int32_t *indices;
  const float *values;
} sps_csr;

/* Opaque host handles. Immutable once prepared; the device data they refer
 * to lives in caller-owned workspaces. */
typedef struct sps_items sps_items;
typedef struct sps_queries sps_queries;

/* ------------------------------------------------------------------ */
/* Items: norms + per-chunk inverted lists                             */
/* ------------------------------------------------------------------ */

/* Byte sizes for sps_prepare. `persistent` holds the prepared corpus and
 * must outlive the handle; `scratch` is only used by sps_prepare itself and
 * may be reused once the prepare's stream work has completed.
 * chunk_size: items per chunk, 1..1048576 (the page uses 8192, §3.3).
 * Pure host arithmetic; no device access. */
sps_status sps_items_workspace_size(int64_t n_items, int64_t dim, int64_t nnz,
                                    int32_t chunk_size, size_t *persistent_bytes,
                                    size_t *scratch_bytes);

/* Prepare an item corpus (asynchronous, stream-ordered):
 *  1. inverse norms inv[i] = fl32(1 / sqrt(sum v^2)) with the sum in float64
 *     over the stored nonzeros in index order (§5.2); 0 for a zero norm;
 *  2. chunk c covers items [c*chunk_size, min((c+1)*chunk_size, n_items))
 *     (§4.4 slicing). Each chunk is cut into slices_per_chunk =
 *     ceil(chunk_size / 1024) slices of slice_size = ceil(chunk_size /
 *     slices_per_chunk) items (the last slice of a chunk may be shorter): a
 *     slice is what one workgroup accumulates on chip;
 *  3. per slice, the inverted lists (the CSC of the slice's items): for every
 *     entry an sps_posting, the slice-local item id and the value
 *     fl32(v / ||item||) rounded once from float64 (0 if the item norm is 0),
 *     grouped by dim in ascending dim order, item ids ascending within each
 *     dim. The lists are located through a per-slice hash index of the dims
 *     the slice holds (dim -> first posting, length), about 32 bytes per
 *     distinct dim, instead of a col_ptr[dim+1] per slice; the canonical
 *     col_ptr can be expanded from it (sps_items_slice_col_ptr);
 *  4. when slices hold at least 512 items: the "heavy" dims, the most
 *     frequent among those held by at least 1/16 of the items (a dim counted
 *     only in the slices where its list holds 1/32 of the slice), in blocks of
 *     32: the first block, and up to three more while a block's dims carry
 *     enough of the expected work (the sum over its dims of (df / n_items)^2
 *     above 0.4, SPS_HEAVY_GAIN overrides); at most 128, SPS_HEAVY_MAX caps
 *     it (and sizes the slab); per slice, their values as dense rows (0 where
 *     an item lacks the dim). This is a speed device; results do not depend
 *     on it beyond rounding (SPS_DENSE=0 turns it off).
 * The item CSR may be released once this stream work has completed.
 * On success *out receives a new handle (free with sps_items_destroy). */
sps_status sps_prepare(const sps_csr *items, int32_t chunk_size, void *persistent,
                       size_t persistent_bytes, void *scratch, size_t scratch_bytes,
                       void *stream, sps_items **out);

/* Sizes of a prepared corpus (pure host): items, dimension, nonzeros, the
 * chunk size and the number of chunks, ceil(n_items / chunk_size) (the
 * chunk loop of §4.4 runs over them). Each output pointer is nullable.
 * Errors: SPS_ERR_INVALID_ARGUMENT for a NULL handle. */
sps_status sps_items_info(const sps_items *h, int64_t *n_items, int64_t *dim, int64_t *nnz,
                          int32_t *chunk_size, int32_t *num_chunks);

/* Slice geometry (see sps_prepare step 2): how each chunk of §4.4 is cut
 * for the device. Slice s of the corpus is slice s % slices_per_chunk of
 * chunk s / slices_per_chunk. Pure host; output pointers nullable; errors:
 * SPS_ERR_INVALID_ARGUMENT for a NULL handle. */
sps_status sps_items_slices(const sps_items *h, int32_t *slice_size, int32_t *slices_per_chunk,
                            int64_t *num_slices);

/* One entry of a slice's inverted lists: the slice-local item id and the
 * value fl32(v / ||item||). Stored together (8 bytes) so that one load
 * fetches both. */
typedef struct {
  uint32_t item;
  float value;
} sps_posting;

/* Device views of one prepared slice (for parity tests and tooling).
 * SYNCHRONOUS: reads the slice's entry range back from the device after
 * synchronising `stream`. post: DEVICE sps_posting[slice_nnz] (the lists in
 * ascending dim order); item_inv_norm: DEVICE float[slice_len] (the slice's
 * first item onwards). */
typedef struct {
  int64_t item_begin;
  int32_t slice_len;
  int32_t slice_nnz;
  const sps_posting *post;
  const float *item_inv_norm;
} sps_slice_view;

sps_status sps_items_slice_view(const sps_items *h, int64_t slice, void *stream,
                                sps_slice_view *view);

/* The slice's canonical CSC column pointer, expanded from its dim index
 * (asynchronous): col_ptr[d] = the number of the slice's entries with a
 * column below d, d = 0..dim (col_ptr[0] = 0, col_ptr[dim] = slice nnz),
 * the layout of a CSC's column pointer (§4.4 slicing; for verification and
 * tools, not used by scoring). col_ptr: DEVICE int32[dim+1], caller-owned.
 * status (nullable): DEVICE int32, zeroed by the caller; bit 1 is set if a
 * list's length in the index disagrees with the next list's start (an
 * inconsistent index). Errors: SPS_ERR_INVALID_ARGUMENT (NULL),
 * SPS_ERR_CHUNK_RANGE (slice out of range). */
sps_status sps_items_slice_col_ptr(const sps_items *h, int64_t slice, int32_t *col_ptr,
                                   int32_t *status, void *stream);

/* The heavy dims chosen by sps_prepare, ascending, at most 128
 * (SYNCHRONOUS: waits for `stream`, then copies 516 bytes back). The page notes that term ids
 * cluster in a dictionary prefix (§3.2, Block-Sparse CSR motivation); the
 * few dims most items hold are scored as dense rows. Writes at most
 * `capacity` dims to `dims` (host, nullable) and their number to *count
 * (host; 0 when the dense rows are off or no dim qualifies). Errors:
 * SPS_ERR_INVALID_ARGUMENT (NULL handle or count), SPS_ERR_HIP. */
sps_status sps_items_heavy_dims(const sps_items *h, void *stream, int32_t *dims,
                                int32_t capacity, int32_t *count);

/* Free the host handle (never the caller's workspaces). NULL is ignored. */
void sps_items_destroy(sps_items *h);

/* ------------------------------------------------------------------ */
/* Queries                                                             */
/* ------------------------------------------------------------------ */

/* Byte size of the query workspace for a query batch scored against the
 * prepared items `items` (the row grouping depends on the item chunk size).
 * Pure host arithmetic. */
sps_status sps_queries_workspace_size(const sps_items *items, int64_t n_rows, int64_t dim,
                                      int64_t nnz, size_t *bytes);

/* Prepare a query batch for the prepared items `items` (asynchronous):
 * inverse norms as for items (§5.2); every row normalised by its float64
 * norm and rounded once to fp32, fl32(q_d / ||q||); values on the items'
 * heavy dims gathered into dense blocks of 16 rows, the rest kept as "light"
 * records (dim, value, row) per group of 16 rows, sorted by dim within the
 * group (so that rows sharing a dim walk its posting list close together).
 * The query CSR may be released once this stream work has
 * completed. The batch can only be scored against `items`. Free the handle
 * with sps_queries_destroy. */
sps_status sps_prepare_queries(const sps_csr *queries, const sps_items *items,
                               void *workspace, size_t workspace_bytes, void *stream,
                               sps_queries **out);

/* The query batch's inverse norms fl32(1 / ||q||) (§5.2), computed by
 * sps_prepare_queries: *inv_norm receives a DEVICE float[n_rows] pointer
 * into the batch's workspace (valid while the workspace is; read it after
 * the prepare's stream work). Errors: SPS_ERR_INVALID_ARGUMENT (NULL). */
sps_status sps_queries_inv_norms(const sps_queries *q, const float **inv_norm);

/* Free the host handle (never the caller's workspace). NULL is ignored. */
void sps_queries_destroy(sps_queries *q);

/* ------------------------------------------------------------------ */
/* Scoring                                                             */
/* ------------------------------------------------------------------ */

/* Score chunk `chunk` (asynchronous): for every query row q and every item
 * j < chunk_len of the chunk,
 *     out[q * ld_out + j] = S[q, item_begin + j]          (float32)
 * computed as sum over the shared dims of fl32(q_d/|q|) * fl32(i_d/|i|)
 * (both rows normalised before the dot; the page divides after it, §4.4 --
 * equal up to rounding). The light dims are summed exactly in 32-bit fixed
 * point (2^-30) after rounding each fp32 product; the heavy dims in fp32 on
 * the matrix cores, then added. Columns chunk_len <= j < ld_out are not
 * touched. out: DEVICE, n_rows * ld_out floats, ld_out >= min(chunk_size,
 * n_items). row_sums (nullable): DEVICE double[n_rows]; row_sums[q] = the
 * float64 sum of the float32 scores written for row q (a per-chunk checksum).
 * No clamping to [-1, 1] is applied. Results are bitwise reproducible.
 * Concurrency: with chunk_size above 1024 the per-slice partial row sums go
 * through a buffer in the query batch's workspace, so calls that pass
 * row_sums for the same sps_queries must be ordered on one stream (calls
 * without row_sums, or on different query batches, may run concurrently). */
sps_status sps_cosine_chunk(const sps_queries *q, const sps_items *items, int32_t chunk,
                            float *out, int64_t ld_out, double *row_sums, void *stream);

/* sps_cosine_chunk for callers that cannot allocate device memory, or would
 * rather not keep a per-batch partial-row-sum buffer in use (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc). Same
 * arguments, results and errors as sps_cosine_chunk, bit for bit; the only
 * difference is where the per-slice partial row sums live (chunk_size above
 * 1024 with row_sums != NULL): in a 4 MiB static device array that the
 * library holds on each GPU it runs on until the process ends, instead of
 * the query batch's workspace. Nothing is allocated by this call. Limit:
 * n_rows * ceil(chunk_size / 1024) <= 524288 when row_sums is given
 * (SPS_ERR_UNSUPPORTED otherwise). All calls of it on one GPU share that
 * array: calls that overlap on one GPU (on different streams, or from
 * several threads without ordering) race and their row sums are
 * unspecified; calls ordered on one stream are fine. */
sps_status sps_cosine_chunk_static(const sps_queries *q, const sps_items *items, int32_t chunk,
                                   float *out, int64_t ld_out, double *row_sums, void *stream);

/* Score chunks [chunk_begin, chunk_end) one after another into the same
 * rotating buffer `out` (the streaming loop of §2.2 and §4.4 with the chunk
 * output kept on the device). row_sums (nullable): DEVICE
 * double[(chunk_end-chunk_begin) * n_rows], chunk-major. */
sps_status sps_cosine_stream(const sps_queries *q, const sps_items *items, int32_t chunk_begin,
                             int32_t chunk_end, float *out, int64_t ld_out, double *row_sums,
                             void *stream);

/* The streaming loop with the output on the host (§2.2, §4.4: each chunk's
 * scores are accumulated into a host output buffer). Chunks [chunk_begin,
 * chunk_end) are scored in turn into the two DEVICE buffers dev_buf0 and
 * dev_buf1 (n_rows * ld_dev floats each, ld_dev >= min(chunk_size, n_items),
 * distinct), alternately, on `stream`; the copy engine moves each chunk into
 * its column block of the host matrix on `copy_stream`, so that the copy of
 * one chunk overlaps the scoring of the next:
 *     host_out[q * ld_host + (item - item_begin)] = S[q, item]
 * for every item of the range, item_begin = chunk_begin * chunk_size.
 * host_out: page-locked HOST memory (hipHostMalloc, or a pinned torch
 * tensor), n_rows * ld_host floats, ld_host >= the number of items in the
 * range; columns past them are not touched. row_sums (nullable): DEVICE
 * double[(chunk_end-chunk_begin) * n_rows], chunk-major, as in
 * sps_cosine_stream. The work completes in `stream` order (the stream waits
 * for the last copy): synchronise `stream` before reading host_out. Both
 * buffers and host_out must stay untouched until then. copy_stream should
 * be a stream other than `stream` (the same one is correct but serialises
 * the copies with the scoring). Errors: SPS_ERR_INVALID_ARGUMENT (NULL or
 * equal buffers, host_out not page-locked, ld too small),
 * SPS_ERR_CHUNK_RANGE, SPS_ERR_OVERFLOW; SPS_ERR_HIP if a runtime call fails
 * (then part of the range may have been enqueued). */
sps_status sps_cosine_stream_host(const sps_queries *q, const sps_items *items,
                                  int32_t chunk_begin, int32_t chunk_end, float *host_out,
                                  int64_t ld_host, float *dev_buf0, float *dev_buf1,
                                  int64_t ld_dev, double *row_sums, void *stream,
                                  void *copy_stream);

/* One score kept by sps_cosine_chunk_threshold: query row, global item
 * index, and the float32 score. */
typedef struct {
  int32_t row;
  int32_t item;
  float score;
} sps_hit;

/* Threshold-filtered output (asynchronous), for the threshold filtering the
 * page's downstream logic applies to the full matrix (§2.3): the scores of
 * chunk `chunk` are computed as in sps_cosine_chunk and every one with
 * S[q, j] >= threshold (compared in float32) is appended as a hit (q,
 * item_begin + j, S) to hits[*count ...]: *count (DEVICE uint64, zeroed by the
 * caller once) is advanced atomically by the number of hits, so successive
 * calls append; hits past `capacity` are counted but not written (the caller
 * compares *count with capacity). The order of hits is unspecified; the set
 * and each score are bitwise reproducible and equal to sps_cosine_chunk's.
 * hits: DEVICE sps_hit[capacity]; row_sums (nullable): DEVICE double[n_rows],
 * the float64 sum of all the chunk's scores of the row, kept or not.
 * Errors: SPS_ERR_INVALID_ARGUMENT (NULL count, negative capacity, NaN
 * threshold), SPS_ERR_CHUNK_RANGE. */
sps_status sps_cosine_chunk_threshold(const sps_queries *q, const sps_items *items, int32_t chunk,
                                      float threshold, sps_hit *hits, int64_t capacity,
                                      uint64_t *count, double *row_sums, void *stream);

/* ------------------------------------------------------------------ */
/* Reduced-precision variant (fp16)                                    */
/* ------------------------------------------------------------------ */

/* The page allows fp16 value data where a loss below 1e-3 is acceptable,
 * with the norms kept in float32 (§5.3). This variant stores each item value
 * as fp16(2^15 * fl32(v / ||item||)) (a 4-byte posting with the slice-local
 * item id) and writes fp16 scores; query values and all norms stay float32
 * and the accumulation is the same as in sps_cosine_chunk. Error: the item
 * values contribute at most 2^-11 * sum_d |q_d i_d| <= 2^-11 (Cauchy-Schwarz
 * on unit rows) and the fp16 output rounding at most 2^-11 for |S| <= 1 +
 * 2^-11, so |S_half - S| < 1e-3 for every score. */

/* Bytes of the workspace for sps_items_enable_half: (nnz + 4) * 4. Pure host. */
sps_status sps_items_half_workspace_size(const sps_items *h, size_t *bytes);

/* Build the 4-byte postings of a prepared corpus (asynchronous, after the
 * sps_prepare work on the same stream). workspace: DEVICE, 16-byte aligned,
 * caller-owned, kept alive while the handle is used for sps_cosine_chunk_half;
 * errors: SPS_ERR_WORKSPACE_TOO_SMALL, SPS_ERR_INVALID_ARGUMENT. */
sps_status sps_items_enable_half(sps_items *h, void *workspace, size_t workspace_bytes,
                                 void *stream);

/* sps_cosine_chunk with fp16 scores (IEEE binary16 bit patterns in `out`,
 * DEVICE uint16[n_rows * ld_out]) computed from the fp16 item values above;
 * row_sums (nullable) = the float64 sum of the fp16 scores written. Requires
 * sps_items_enable_half (SPS_ERR_INVALID_ARGUMENT otherwise). Bitwise
 * reproducible. */
sps_status sps_cosine_chunk_half(const sps_queries *q, const sps_items *items, int32_t chunk,
                                 uint16_t *out, int64_t ld_out, double *row_sums, void *stream);

/* ------------------------------------------------------------------ */
/* Block-Sparse CSR codec                                              */
/* ------------------------------------------------------------------ */

/* Compressed column indices (§3.2: Block-Sparse CSR). A column d is the pair
 * (block = d / 1024, offset = d % 1024). Row by row, the block ids (ascending
 * in a canonical row) are stored as differences from the previous entry's
 * block id, the first from 0, each as an unsigned base-128 varint (7 value
 * bits per byte, least significant group first, the high bit set on every
 * byte of a value but its last: 1 byte below 128, 2 below 16384, 3 for any
 * int32 column). The 10-bit offsets are packed in entry order over the whole
 * matrix, least significant bit first: entry k at bits 10k .. 10k + 9 of the
 * byte stream. Where the page leaves it open: differences restart at each
 * row, so rows decode independently; the varint bytes of row r start at
 * bptr[r] (a second row pointer, since they cannot be located by entry).
 * indptr and values are the CSR's. nnz is limited to (2^31 - 1) / 3. */
typedef struct {
  int64_t n_rows;
  int64_t n_cols;
  int64_t nnz;
  const int32_t *indptr;   /* DEVICE int32[n_rows + 1]: entry positions (the CSR's) */
  const int32_t *bptr;     /* DEVICE int32[n_rows + 1]: byte positions in `blocks` */
  const uint8_t *blocks;   /* DEVICE uint8[block_bytes]: the block-id varints */
  int64_t block_bytes;     /* = bptr[n_rows] */
  const uint8_t *offsets;  /* DEVICE uint8[offsets_bytes]: the packed 10-bit offsets */
  int64_t offsets_bytes;   /* >= ceil(10 nnz / 8) */
  const float *values;     /* DEVICE float[nnz] (the CSR's) */
} sps_bsc;

/* Bytes of the offset stream for nnz entries: ceil(10 nnz / 8) rounded up to
 * a multiple of 4 (sps_bsc_encode writes whole 32-bit words; the tail bits
 * are zero). Pure host. SPS_ERR_OVERFLOW for nnz above the codec's limit
 * (floor((2^31 - 1) / 3), the limit of sps_bsc_encode_sizes). */
sps_status sps_bsc_offsets_bytes(int64_t nnz, size_t *bytes);

/* First half of the encoder (SYNCHRONOUS): checks that m is canonical (as
 * sps_validate_csr; scratch: DEVICE, >= 64 bytes, 8-byte aligned), writes the
 * row byte pointers bptr (DEVICE int32[n_rows + 1]) and returns the size of
 * the varint stream in *block_bytes. Errors: SPS_ERR_BAD_CSR,
 * SPS_ERR_OVERFLOW (nnz above the limit), SPS_ERR_INVALID_ARGUMENT. */
sps_status sps_bsc_encode_sizes(const sps_csr *m, int32_t *bptr, void *scratch, void *stream,
                                int64_t *block_bytes);

/* Second half (asynchronous): the varint stream into blocks (DEVICE
 * uint8[block_bytes], block_bytes from sps_bsc_encode_sizes for the same m)
 * and the offset stream into offsets (DEVICE, 4-byte aligned, offsets_bytes
 * >= sps_bsc_offsets_bytes(nnz)). Nothing is written past either size.
 * Errors: SPS_ERR_WORKSPACE_TOO_SMALL (offsets), SPS_ERR_INVALID_ARGUMENT. */
sps_status sps_bsc_encode(const sps_csr *m, const int32_t *bptr, uint8_t *blocks,
                          int64_t block_bytes, uint8_t *offsets, int64_t offsets_bytes,
                          void *stream);

/* Decode (asynchronous) the column indices of b into indices (DEVICE
 * int32[nnz]); with b->indptr and b->values they form the CSR that was
 * encoded, ready for sps_prepare (which may then drop them). Any contents
 * are safe to decode: no access leaves the sizes given. If the encoding is
 * malformed (a row's bytes do not hold exactly its entries, or a value of
 * more than 3 bytes), *status (DEVICE int32, nullable, zeroed by the caller)
 * gets bit 1 and the indices are unspecified. */
sps_status sps_bsc_decode(const sps_bsc *b, int32_t *indices, int32_t *status, void *stream);

/* ------------------------------------------------------------------ */
/* Stand-alone pieces                                                  */
/* ------------------------------------------------------------------ */

/* Inverse row norms of any CSR (asynchronous): inv_norm DEVICE float[n_rows],
 * fl32(1/sqrt(sum v^2)), float64 sum in index order, 0 for a zero norm
 * (§5.2). */
sps_status sps_row_inv_norms(const sps_csr *rows, float *inv_norm, void *stream);

/* Full canonical-CSR check (SYNCHRONOUS), the precondition of the page's
 * merge (§3.1 note: strictly ordered indices). scratch: DEVICE, >= 64 bytes.
 * Returns SPS_OK, or SPS_ERR_BAD_CSR with *first_bad_row (nullable) set to
 * the lowest offending row (0 for a fault in indptr[0] or indptr[n_rows])
 * and *reason (nullable): 1 indptr, 2 order/duplicate, 3 index range,
 * 4 non-finite value. */
sps_status sps_validate_csr(const sps_csr *m, void *scratch, void *stream,
                            int64_t *first_bad_row, int32_t *reason);

/* A static English name for a status ("unknown status" for other values). */
const char *sps_status_string(sps_status s);
/* The detail of the calling thread's last failed call (thread-local; empty
 * until a call fails; overwritten by the next failure on the thread). */
const char *sps_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* SPS_H */
