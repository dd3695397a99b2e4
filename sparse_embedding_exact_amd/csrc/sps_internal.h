// sps_internal.h -- constants, geometry and launchers shared by the C-ABI
// layer (sps_api.hip) and the kernel files (sps_prepare.hip, sps_score.hip).
// Not part of the public interface (include/sps.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sps {

// flags block (device, 16 int32): [0] structural fault bits (1 indptr,
// 4 index range), [1] other fault bits (2 order/duplicate, 8 non-finite),
// [2..3] uint64 min key (row << 3 | reason code) of the first faulty row.
constexpr int kFlagsInts = 16;

// Query rows per score workgroup and the widest item slice one workgroup
// accumulates on chip: 16 rows x 1024 items x 4 B = 64 KiB of LDS, so two
// workgroups (8 waves each) share a CU's 160 KiB.
constexpr int kRows = 16;
constexpr int kSliceMax = 1024;
constexpr int kScoreThreads = 512;
// zeroed postings past the end of the posting array: the score kernel reads
// postings in pairs, so the pair of a list's last posting stays readable
constexpr int kPostPad = 2;
// the same for the 4-byte postings of the reduced-precision variant, read
// four at a time
constexpr int kPostPad4 = 4;

// Dense path for heavy dims: blocks of kHeavyBlock dims (the depth of one
// v_mfma_f32_16x16x32_f16), at most kHeavyBlocksMax of them, taken from the
// dims whose item document frequency is at least n_items / kHeavyFracInv;
// only for slices of at least kDenseMinSlice items. The prepare takes one
// block, and each further block while it moves enough of the expected
// sparse work onto the matrix cores (see heavy_rank_kernel).
constexpr int kHeavyBlock = 32;
constexpr int kHeavyBlocksMax = 4;
constexpr int kHeavyMax = kHeavyBlock * kHeavyBlocksMax;
constexpr int kHeavyFracInv = 16;
// The walk's cost of a further block's dims must exceed this many (query
// entry, posting) products per score to take that block (heavy_rank_kernel):
// a block of 32 dims on the matrix cores costs about as much as 0.4 such
// products of the sparse walk per score (both measured on gfx950 at the
// pages' shape: 0.17 and 0.8 ps per score and per product).
constexpr float kHeavyBlockGain = 0.4f;
constexpr int kDenseMinSlice = 512;

// 32-bit fixed point of the on-chip accumulators: 30 fraction bits.
constexpr float kFixScale = 1073741824.0f;        // 2^30
constexpr float kFixInv = 9.313225746154785e-10f;  // 2^-30

// Item chunks of C items (the unit of output) are cut into n_sub slices of
// S items (the unit of the inverted lists and of one workgroup's LDS).
struct Geom {
  int64_t n_items;
  int32_t C, n_sub, S, num_chunks;
  __host__ __device__ int64_t num_slices() const { return (int64_t)num_chunks * n_sub; }
  __host__ __device__ int64_t chunk_begin(int64_t c) const {
    const int64_t b = c * C;
    return b < n_items ? b : n_items;
  }
  __host__ __device__ int64_t chunk_end(int64_t c) const {
    const int64_t e = (c + 1) * C;
    return e < n_items ? e : n_items;
  }
  __host__ __device__ int64_t slice_begin(int64_t s) const {
    const int64_t c = s / n_sub, k = s % n_sub;
    const int64_t b = c * C + k * S, ce = chunk_end(c);
    return b < ce ? b : ce;
  }
  __host__ __device__ int64_t slice_end(int64_t s) const {
    const int64_t c = s / n_sub, k = s % n_sub;
    const int64_t e = c * C + (k + 1) * S, ce = chunk_end(c);
    return e < ce ? e : ce;
  }
  __host__ __device__ int64_t slice_of(int64_t i) const {
    const int64_t c = i / C;
    return c * n_sub + (i - c * C) / S;
  }
};

inline Geom make_geom(int64_t n_items, int32_t chunk_size) {
  Geom g;
  g.n_items = n_items;
  g.C = chunk_size;
  g.n_sub = (chunk_size + kSliceMax - 1) / kSliceMax;
  g.S = (chunk_size + g.n_sub - 1) / g.n_sub;
  g.num_chunks = (int32_t)((n_items + chunk_size - 1) / chunk_size);
  return g;
}
// Heavy-dim values are kept as split fp16 pairs for the matrix cores: with
// X = 2^15 x (exact), hi = fp16(X) and lo = fp16((X - hi) * 2048), so that
// X = hi + lo / 2048 up to 2^-22 |X|. Items (and query rows) are stored per
// block of kHeavyBlock dims in tiles of 16: a tile is kTileHalves halves,
// the hi part then the lo part, each [dim group of 8][item of the tile][8
// dims] -- exactly the per-lane operand order of v_mfma_f32_16x16x32_f16
// (lane l = item l%16, dim group l/16), so one 16-byte load per lane reads
// 1 KiB of contiguous memory. Dims past the heavy count are zero. Heavy dim
// k (its position in the ascending heavy list) is dim k % kHeavyBlock of
// block k / kHeavyBlock.
constexpr int kHeavyRec = 2 * kHeavyBlock;  // halves per item and block
constexpr int kTileHalves = 16 * kHeavyRec;
// The scale 2^15 makes a product of two scaled values 2^30 times the product
// of the values -- the fixed-point scale of the accumulators -- so the dense
// sums need no rescaling; |x| <= 1 keeps X within fp16's range (|X| <=
// 32768, |lo| <= 16384), and values down to 2^-29 stay normal in fp16.
constexpr float kHeavyScale = 32768.0f;  // X = x * 2^15
constexpr float kLoScale = 2048.0f;    // lo = (X - hi) * 2048
// position of (item j, dim h of the block, part 0 hi / 1 lo) from its
// tile's start
__host__ __device__ inline int heavy_tile_index(int j, int h, int part) {
  return part * (16 * kHeavyBlock) + ((h & (kHeavyBlock - 1)) >> 3) * 128 + (j & 15) * 8 +
         (h & 7);
}
// blocks of kHeavyBlock dims needed for `cap` heavy dims
__host__ __device__ inline int32_t heavy_blocks(int32_t cap) {
  return (cap + kHeavyBlock - 1) / kHeavyBlock;
}
__device__ inline void split_fp16(float x, uint16_t &hi, uint16_t &lo) {
  const float X = x * kHeavyScale;
  const _Float16 h = (_Float16)X;
  const _Float16 l = (_Float16)((X - (float)h) * kLoScale);
  hi = __builtin_bit_cast(uint16_t, h);
  lo = __builtin_bit_cast(uint16_t, l);
}

// Item pitch of a slice's heavy-dim slab: a whole number of 128-item groups
// (one wave's share in the dense part).
__host__ __device__ inline int32_t slab_pitch(int32_t S) { return (S + 127) / 128 * 128; }

// ---- per-slice dim index: dim -> (first posting, list length) ----
// A slice's inverted lists are the CSC of its items: lists in ascending dim
// order, located by col_ptr[dim + 1]. Only the dims the slice holds have a
// non-empty list, so instead of col_ptr (4 (dim + 1) bytes per slice, mostly
// repeats) each slice keeps an open-addressing hash table of its non-empty
// lists, small enough to stay in the L2 of the XCD that walks the slice.
//  - info[s] = (first bucket, bucket count nb, wide, distinct dims); nb =
//    max(1, 2 * distinct), so at most a quarter of the slots (narrow) or half
//    of the buckets (wide) are used and a probe chain always ends (about 19
//    lookups in 20 end in their home bucket);
//  - a bucket is 16 bytes: two 8-byte slots (key = dim, value), or, for a
//    "wide" slice (more than 2^22 entries), one key per bucket with the start
//    and the length in separate words;
//  - narrow value = start | (length - 1) << 22 (start is slice-relative, a
//    length is at most the slice's item count, <= 1024);
//  - home bucket = floor(nb * fib(d) / 2^32) with fib(d) = (d * 0x9E3779B1)
//    mod 2^32 (Fibonacci hashing); linear probing by bucket.
// Empty slots hold all ones (no dim is 2^32 - 1). The lookup result is
// exact; the placement of keys in the table depends on insertion order and
// is never observed.
constexpr uint32_t kDimEmpty = 0xFFFFFFFFu;
constexpr int kStartBits = 22;
constexpr int64_t kNarrowMaxNnz = 1ll << kStartBits;
constexpr int kBucketsPerDim = 2;
__host__ __device__ inline uint32_t dim_bucket(uint32_t d, uint32_t nb) {
  const uint32_t h = d * 0x9E3779B1u;
  return (uint32_t)(((uint64_t)h * nb) >> 32);
}
// One bucket's verdict for dim d: 1 found (start, len set), 0 absent, -1 look
// in the next bucket.
__device__ __forceinline__ int dim_probe(uint4 e, uint32_t d, bool wide, int32_t &start,
                                         int32_t &len) {
  if (wide) {
    if (e.x == d) {
      start = (int32_t)e.y;
      len = (int32_t)e.w;
      return 1;
    }
    return e.x == kDimEmpty ? 0 : -1;
  }
  if (e.x == d || e.z == d) {
    const uint32_t v = e.x == d ? e.y : e.w;
    start = (int32_t)(v & ((1u << kStartBits) - 1u));
    len = (int32_t)(v >> kStartBits) + 1;
    return 1;
  }
  return (e.x == kDimEmpty || e.z == kDimEmpty) ? 0 : -1;
}
// the full lookup (a chain is never longer than nb buckets)
__device__ __forceinline__ bool dim_lookup(const uint4 *__restrict__ tab, int4 info, uint32_t d,
                                           int32_t &start, int32_t &len) {
  const uint32_t nb = (uint32_t)info.y;
  uint32_t b = dim_bucket(d, nb);
  for (uint32_t k = 0; k < nb; ++k) {
    const int r = dim_probe(tab[(int64_t)info.x + b], d, info.z != 0, start, len);
    if (r >= 0) return r == 1;
    b = b + 1 == nb ? 0u : b + 1;
  }
  return false;
}
// Row pitch (ints) of the score kernel's LDS accumulators: the slab pitch
// plus 4, so that rows start 16 bytes apart modulo the LDS bank period.
__host__ __device__ inline int32_t acc_pitch(int32_t S) { return slab_pitch(S) + 4; }
inline bool dense_slice_ok(int32_t S) { return S >= kDenseMinSlice; }

hipError_t launch_fill_i32(int32_t *p, int64_t n, int32_t v, hipStream_t s);
// inclusive scan in place over a[0..n) (one workgroup)
hipError_t launch_scan_inplace(int32_t *a, int64_t n, hipStream_t s);
hipError_t launch_csr_check(int64_t n_rows, int64_t n_cols, int64_t nnz, const int32_t *indptr,
                            const int32_t *indices, const float *values, int full,
                            int32_t *flags, hipStream_t s);
hipError_t launch_row_norms(int64_t n_rows, int64_t nnz, const int32_t *indptr,
                            const float *values, const int32_t *flags, float *inv32,
                            double *norm64, hipStream_t s);

// ---- items: per-slice inverted lists (+ dense slabs of heavy dims) ----
struct ItemsDev {
  Geom g;
  int64_t dim, nnz;
  bool dense;           // build heavy-dim slabs
  int32_t heavy_cap;    // at most this many heavy dims (<= kHeavyMax)
  int64_t slab_bstride; // halves from one block's slab to the next's
  float heavy_gain;     // a further block needs this many products per score (heavy_rank_kernel)
  const int32_t *indptr, *indices;
  const float *values;
  float *inv_norm;      // persistent, n_items
  int4 *dinfo;          // persistent, num_slices + 1: dim index per slice (info[ns].x = buckets)
  uint4 *dtab;          // persistent, 2 nnz + num_slices buckets (the used prefix is filled)
  uint2 *post;          // persistent, nnz + kPostPad: (slice-local item id, value bits)
  int32_t *slice_base;  // persistent, num_slices + 1
  int32_t *heavy;       // persistent, kHeavyMax + 1: heavy dims ascending, then their count
  uint16_t *slab;       // persistent, [heavy_blocks(heavy_cap)][num_slices][pitch / 16 tiles]
                        // split fp16 (dense only)
  int32_t *flags;       // scratch
  double *norm64;       // scratch, n_items
  int32_t *skey[2];     // scratch, nnz each: columns during the radix sort (sorted: skey[0])
  uint2 *spay;          // scratch, nnz: (item, value) during the radix sort
  int32_t *gdf;         // scratch, kGdfStripes * dim (dense only)
  int32_t *hsel;        // scratch, kHeavySelInts (dense only): heavy-dim candidates
};
constexpr int kHeavySelInts = 33 + 2 * 2048;
// The heavy-dim document frequencies are counted in this many copies of the
// dim-sized array (slice s adds to copy s % kGdfStripes), then summed: the
// most frequent dims have a long list in nearly every slice, and one counter
// per dim would take all of those atomic adds in turn.
constexpr int kGdfStripes = 16;
hipError_t launch_prepare_items(const ItemsDev &d, hipStream_t s);
// col_ptr[0..dim] of slice `slice` expanded from its dim index; *status |= 1
// (nullable) where a list's length disagrees with the next list's start
hipError_t launch_expand_col_ptr(int64_t dim, const int4 *dinfo, const uint4 *dtab,
                                 const int32_t *slice_base, int64_t slice, int32_t *col_ptr,
                                 int32_t *status, hipStream_t s);
// 4-byte postings (item | fp16(2^15 value) << 16) from the prepared 8-byte
// ones, plus kPostPad4 zero entries
hipError_t launch_pack_half(const uint2 *post, int64_t nnz, uint32_t *post4, hipStream_t s);

// ---- queries ----
struct QueriesDev {
  int64_t n_rows, dim, nnz;
  int32_t n_groups;      // ceil(n_rows / kRows)
  bool dense;
  const int32_t *indptr, *indices;
  const float *values;
  const int32_t *heavy;  // the items' heavy dims (dense only)
  int32_t qh_gstride;    // halves per row group in qh: heavy_blocks(items' cap) tiles
  int32_t *flags;
  float *inv_norm;       // n_rows
  double *norm64;        // n_rows
  int32_t *lptr;         // n_rows + 1: light (non-heavy) entries per row, prefix
  uint3 *lrec;           // nnz: (dim, bits of fl32(q / |q|) * 2^30, row within its group)
  uint16_t *qh;          // [n_groups][blocks] tiles of split fp16: fl32(q / |q|) on heavy dims
};
hipError_t launch_prepare_queries(const QueriesDev &d, hipStream_t s);

// ---- scoring ----
// output modes of the score kernel: fp32 scores, fp16 scores (reduced-precision
// variant), or only the scores >= a threshold as (row, item, score) hits
enum ScoreMode : int32_t { kModeExact = 0, kModeHalf = 1, kModeThreshold = 2 };
struct ScoreArgs {
  ScoreMode mode;
  Geom g;
  int64_t dim, n_q;
  int32_t n_groups;
  int32_t chunk;
  bool dense;
  const int32_t *lptr;
  const uint3 *lrec;          // light entries: (dim, value bits, row in group)
  const uint16_t *qh;         // [row groups][blocks] tiles of split fp16 (dense only)
  int32_t qh_gstride;         // halves per row group in qh
  const int4 *dinfo;          // dim index of every slice
  const uint4 *dtab;
  const uint2 *post;          // all slices: (slice-local item id, value bits)
  const uint32_t *post4;      // reduced-precision variant: item | fp16(2^15 value) << 16
  const int32_t *slice_base;
  const int32_t *heavy;
  const uint16_t *slab;       // [blocks][slices][pitch / 16] tiles of split fp16 (dense only)
  int64_t slab_bstride;       // halves from one block's slab to the next's
  int32_t heavy_blocks;       // blocks the slab and qh hold (the heavy count never needs more)
  int32_t pitch;
  float *out;
  uint16_t *out16;            // fp16 output of the reduced-precision variant (else null)
  int3 *hits;                 // threshold output (row, item, score bits) (else null)
  int64_t hit_cap;
  unsigned long long *hit_count;
  float threshold;
  int64_t ld;
  double *rs_part;            // n_sub * n_q partial row sums (nullable)
  double *row_sums;           // n_q (nullable)
};
// ---- Block-Sparse CSR codec (sps_bsc.hip) ----
// bptr[0] = 0, bptr[r + 1] = bytes of rows 0..r's block-id varints
hipError_t launch_bsc_row_bytes(int64_t n_rows, int64_t nnz, const int32_t *indptr,
                                const int32_t *indices, int32_t *bptr, hipStream_t s);
hipError_t launch_bsc_encode(int64_t n_rows, int64_t nnz, const int32_t *indptr,
                             const int32_t *indices, const int32_t *bptr, uint8_t *blocks,
                             int64_t block_bytes, uint32_t *offset_words, int64_t n_words,
                             hipStream_t s);
// status |= 1 for a malformed encoding
hipError_t launch_bsc_decode(int64_t n_rows, int64_t nnz, const int32_t *indptr,
                             const int32_t *bptr, int64_t n_bytes, const uint8_t *blocks,
                             const uint8_t *offsets, int32_t *indices, int32_t *status,
                             hipStream_t s);

size_t score_lds_bytes(int32_t S);
hipError_t launch_score(const ScoreArgs &a, hipStream_t s);

}  // namespace sps
