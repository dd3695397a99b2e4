// sps_prepare.hip -- gfx950 kernels that prepare items and queries for
// exact all-pairs sparse cosine.
//
// Page cited throughout: "稀疏嵌入批量相似度计算的工程化实践"
// (Engineering practice of bulk similarity for sparse embeddings).
//
//   csr_check_kernel     §3.1 note: canonical CSR (strictly ordered indices)
//   row_norm_kernel      §5.2 detail one: L2 norm from the stored nonzeros
//   csc_* kernels        per-slice inverted lists; chunk slicing as in §4.4
//   heavy_* / slab_*     dense rows of the few dims most items hold
//   light_* kernels      query rows split into heavy values and the rest,
//                        each row group's light records sorted by dim
//
// All kernels are wave64. Device-side guards keep every access inside the
// buffers the host sized, whatever the CSR contents: the prepare calls run
// csr_check_kernel first, and every later kernel exits when it found a
// structural fault (the dim index then holds no lists).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "sps_device.h"
#include "sps_internal.h"

namespace sps {

// ---------------------------------------------------------------------------
// small utilities
// ---------------------------------------------------------------------------

// p[0..n) = v: 16-byte stores over the aligned middle, the (at most three)
// ints before it and after it by the first workgroup
__global__ void fill_i32_kernel(int32_t *__restrict__ p, int64_t n, int32_t v) {
  const int64_t lead = (int64_t)((16u - (uint32_t)(reinterpret_cast<uintptr_t>(p) & 15u)) & 15u) / 4;
  const int64_t h = lead < n ? lead : n;
  const int64_t n4 = (n - h) / 4;
  int4 *const p4 = reinterpret_cast<int4 *>(p + h);
  const int4 v4 = make_int4(v, v, v, v);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) p4[i] = v4;
  if (blockIdx.x == 0 && threadIdx.x < 4) {
    const int64_t k = threadIdx.x;
    if (k < h) p[k] = v;
    if (h + 4 * n4 + k < n) p[h + 4 * n4 + k] = v;
  }
}

hipError_t launch_fill_i32(int32_t *p, int64_t n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  // (a bounded grid: a launch of many small workgroups is paced by their dispatch)
  int64_t blocks = (n / 4 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

// Inclusive scan in place over a[0..n), in blocks of kScanBlock values (1024
// threads, eight consecutive values each): every block scanned on its own;
// then one workgroup makes each block's last value final (the running sum of
// the blocks' totals); then every block after the first adds the previous
// block's last value to its others. No scratch: the block totals travel in
// the array itself.
constexpr int kScanNT = 1024, kScanPer = 8, kScanBlock = kScanNT * kScanPer;

__global__ __launch_bounds__(kScanNT) void scan_blocks_kernel(int32_t *__restrict__ a, int64_t n) {
  __shared__ int32_t ws[kScanNT / 64];
  const int64_t j0 = (int64_t)blockIdx.x * kScanBlock + (int64_t)threadIdx.x * kScanPer;
  int32_t v[kScanPer];
#pragma unroll
  for (int e = 0; e < kScanPer; ++e) v[e] = j0 + e < n ? a[j0 + e] : 0;
#pragma unroll
  for (int e = 1; e < kScanPer; ++e) v[e] += v[e - 1];
  int32_t tot;
  const int32_t off = block_incl_scan_1b<kScanNT>(v[kScanPer - 1], ws, &tot) - v[kScanPer - 1];
#pragma unroll
  for (int e = 0; e < kScanPer; ++e)
    if (j0 + e < n) a[j0 + e] = off + v[e];
}

// a[last of block b] += the totals of blocks 0 .. b-1 (one workgroup)
__global__ __launch_bounds__(kScanNT) void scan_tops_kernel(int32_t *__restrict__ a, int64_t n) {
  __shared__ int32_t ws[2][kScanNT / 64];
  const int64_t nb = (n + kScanBlock - 1) / kScanBlock;
  int32_t carry = 0;
  int par = 0;
  for (int64_t b0 = 0; b0 < nb; b0 += kScanNT) {
    const int64_t b = b0 + threadIdx.x;
    const int64_t last = b < nb ? ((b + 1) * kScanBlock < n ? (b + 1) * kScanBlock : n) - 1 : 0;
    const int32_t v = b < nb ? a[last] : 0;
    int32_t tot;
    const int32_t incl = block_incl_scan_1b<kScanNT>(v, ws[par], &tot);
    par ^= 1;  // (alternate buffers: one barrier per step suffices)
    if (b < nb) a[last] = carry + incl;
    carry += tot;
  }
}

// block b >= 1: every value but its last += the previous block's last value
__global__ __launch_bounds__(256) void scan_add_kernel(int32_t *__restrict__ a, int64_t n) {
  const int64_t b = blockIdx.x + 1;
  const int64_t first = b * kScanBlock;
  const int64_t last = ((b + 1) * kScanBlock < n ? (b + 1) * kScanBlock : n) - 1;
  const int32_t off = a[first - 1];
  for (int64_t j = first + threadIdx.x; j < last; j += 256) a[j] += off;
}

hipError_t launch_scan_inplace(int32_t *a, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t nb = (n + kScanBlock - 1) / kScanBlock;
  hipLaunchKernelGGL(scan_blocks_kernel, dim3((unsigned)nb), dim3(kScanNT), 0, s, a, n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nb == 1) return e;
  hipLaunchKernelGGL(scan_tops_kernel, dim3(1), dim3(kScanNT), 0, s, a, n);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(scan_add_kernel, dim3((unsigned)(nb - 1)), dim3(256), 0, s, a, n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// CSR check. flags layout in sps_internal.h.
// bit: flag bit (1 indptr, 4 index range -> structural; 2 order, 8 non-finite)
// code: reason code kept with the row in the min key (1 indptr, 2 order,
// 3 index range, 4 non-finite).
// ---------------------------------------------------------------------------

__device__ __forceinline__ void report(int32_t *flags, int64_t row, int bit, int code) {
  if (bit == 1 || bit == 4) atomicOr(&flags[0], bit);
  else atomicOr(&flags[1], bit);
  const unsigned long long key = ((unsigned long long)row << 3) | (unsigned long long)code;
  atomicMin(reinterpret_cast<unsigned long long *>(flags + 2), key);
}

// Rows are checked as in a plain loop over each row. A workgroup whose 256
// row pointers are all in order and in range reads its rows' entries, one
// contiguous range, with coalesced loads: for the index-range check alone,
// entry by entry (an index out of range is charged to its row, found by a
// binary search of the row pointers; a row's later bad indices add nothing
// to what its first one reported), for the full check through LDS windows,
// each thread then walking its own row in order.
constexpr int kCheckWin = 4096;

__global__ __launch_bounds__(256) void csr_check_kernel(int64_t n_rows, int64_t n_cols,
                                                        int64_t nnz,
                                                        const int32_t *__restrict__ indptr,
                                                        const int32_t *__restrict__ indices,
                                                        const float *__restrict__ values,
                                                        int full, int32_t *flags) {
  __shared__ int32_t s_d[kCheckWin];
  __shared__ float s_x[kCheckWin];
  const int64_t r0 = (int64_t)blockIdx.x * 256;
  const int64_t r = r0 + threadIdx.x;
  if (r == 0) {
    if (indptr[0] != 0) report(flags, 0, 1, 1);
    if ((int64_t)indptr[n_rows] != nnz) report(flags, n_rows > 0 ? n_rows - 1 : 0, 1, 1);
  }
  int64_t b = 0, e = 0;
  bool ok = true;
  if (r < n_rows) {
    b = indptr[r];
    e = indptr[r + 1];
    ok = 0 <= b && b <= e && e <= nnz;
    if (!ok) {
      report(flags, r, 1, 1);
      b = e = 0;
    }
  }
  int32_t prev = -1;
  bool live = true;  // no index out of range found yet in this row
  auto check = [&](int64_t r_, int32_t d, float x) {
    if (!live) return;
    if (d < 0 || (int64_t)d >= n_cols) {
      report(flags, r_, 4, 3);
      live = false;
      return;
    }
    if (full) {
      if (d <= prev) report(flags, r_, 2, 2);
      if (!isfinite(x)) report(flags, r_, 8, 4);
    }
    prev = d;
  };
  if (__syncthreads_and(ok)) {
    const int64_t r1 = r0 + 256 < n_rows ? r0 + 256 : n_rows;
    const int64_t vb = r0 < n_rows ? indptr[r0] : 0, ve = r0 < n_rows ? indptr[r1] : 0;
    if (!full) {
      // (eight loads in flight per thread)
      for (int64_t k0 = vb + threadIdx.x; k0 < ve; k0 += 8 * 256) {
        int32_t dd[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) dd[u] = k0 + u * 256 < ve ? indices[k0 + u * 256] : 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int64_t k = k0 + u * 256;
          if (k < ve && (dd[u] < 0 || (int64_t)dd[u] >= n_cols)) {
            // the row holding entry k: the last row of the group starting at or before it
            int64_t lo = r0, hi = r1;
            while (hi - lo > 1) {
              const int64_t mid = (lo + hi) >> 1;
              if ((int64_t)indptr[mid] <= k) lo = mid;
              else hi = mid;
            }
            report(flags, lo, 4, 3);
          }
        }
      }
      return;
    }
    for (int64_t w0 = vb; w0 < ve; w0 += kCheckWin) {
      const int64_t w1 = w0 + kCheckWin < ve ? w0 + kCheckWin : ve;
      __syncthreads();  // the previous window has been read
      for (int64_t k = w0 + threadIdx.x; k < w1; k += 256) {
        s_d[k - w0] = indices[k];
        if (full) s_x[k - w0] = values[k];
      }
      __syncthreads();
      const int64_t kb = b > w0 ? b : w0, ke = e < w1 ? e : w1;
      for (int64_t k = kb; k < ke; ++k) check(r, s_d[k - w0], full ? s_x[k - w0] : 0.0f);
    }
  } else {
    for (int64_t k = b; k < e; ++k) check(r, indices[k], full ? values[k] : 0.0f);
  }
}

hipError_t launch_csr_check(int64_t n_rows, int64_t n_cols, int64_t nnz, const int32_t *indptr,
                            const int32_t *indices, const float *values, int full,
                            int32_t *flags, hipStream_t s) {
  hipError_t e = launch_fill_i32(flags, 2, 0, s);
  if (e != hipSuccess) return e;
  e = launch_fill_i32(flags + 2, 2, -1, s);  // min key starts at all ones
  if (e != hipSuccess) return e;
  const int64_t blocks = (n_rows + 1 + 255) / 256;
  hipLaunchKernelGGL(csr_check_kernel, dim3((unsigned)blocks), dim3(256), 0, s, n_rows, n_cols,
                     nnz, indptr, indices, values, full, flags);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Row norms (§5.2): float64 sum of squares in stored order; fl32(1/sqrt(.)).
// v*v is exact in float64 for a float32 v, so the sum only rounds at the adds.
// ---------------------------------------------------------------------------

// A workgroup takes 256 consecutive rows. When their row pointers are in
// order and in range, their values are one contiguous range of the CSR; it
// is staged through LDS in windows of kNormWin values with coalesced loads,
// and each thread adds its row's squares from LDS in index order, so the sum
// is the same sequence of float64 adds as a plain loop over the row (which
// is what a workgroup with a malformed row pointer does, over the clamped
// row).
constexpr int kNormWin = 4096;

__global__ __launch_bounds__(256) void row_norm_kernel(int64_t n_rows, int64_t nnz,
                                                       const int32_t *__restrict__ indptr,
                                                       const float *__restrict__ values,
                                                       const int32_t *__restrict__ flags,
                                                       float *__restrict__ inv32,
                                                       double *__restrict__ norm64) {
  __shared__ float s_v[kNormWin];
  const int64_t r0 = (int64_t)blockIdx.x * 256;
  const int64_t r = r0 + threadIdx.x;
  const int64_t r1 = r0 + 256 < n_rows ? r0 + 256 : n_rows;
  const bool bad = flags != nullptr && flags[0] != 0;  // uniform
  double sum = 0.0;
  if (!bad) {
    int64_t b = 0, e = 0;
    bool ok = true;
    if (r < n_rows) {
      const int64_t pb = indptr[r], pe = indptr[r + 1];
      ok = 0 <= pb && pb <= pe && pe <= nnz;
      b = clamp64(pb, 0, nnz);
      e = clamp64(pe, b, nnz);
    }
    if (__syncthreads_and(ok)) {
      const int64_t vb = indptr[r0], ve = indptr[r1];
      for (int64_t w0 = vb; w0 < ve; w0 += kNormWin) {
        const int64_t w1 = w0 + kNormWin < ve ? w0 + kNormWin : ve;
        __syncthreads();  // the previous window has been read
        for (int64_t k = w0 + threadIdx.x; k < w1; k += 256) s_v[k - w0] = values[k];
        __syncthreads();
        const int64_t kb = b > w0 ? b : w0, ke = e < w1 ? e : w1;
        for (int64_t k = kb; k < ke; ++k) {
          const double v = (double)s_v[k - w0];
          sum += v * v;
        }
      }
    } else {
      for (int64_t k = b; k < e; ++k) {
        const double v = (double)values[k];
        sum += v * v;
      }
    }
  }
  if (r >= n_rows) return;
  const double n = sqrt(sum);
  if (norm64) norm64[r] = n;
  inv32[r] = (n > 0.0) ? (float)(1.0 / n) : 0.0f;
}

hipError_t launch_row_norms(int64_t n_rows, int64_t nnz, const int32_t *indptr,
                            const float *values, const int32_t *flags, float *inv32,
                            double *norm64, hipStream_t s) {
  if (n_rows <= 0) return hipSuccess;
  const int64_t blocks = (n_rows + 255) / 256;
  hipLaunchKernelGGL(row_norm_kernel, dim3((unsigned)blocks), dim3(256), 0, s, n_rows, nnz,
                     indptr, values, flags, inv32, norm64);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-slice inverted lists. Chunk c holds items [c*C, min((c+1)*C, n))
// (§4.4 slicing); it is cut into n_sub slices of S items (Geom). A slice's
// entries are indptr[first item] .. indptr[last item + 1], and its inverted
// lists occupy that same entry range of the posting array, with item ids
// local to the slice, ascending within each column: the unique CSC of the
// slice (the kernels below build it with a stable sort, so no order of
// concurrent work can change it).
// ---------------------------------------------------------------------------

__global__ void slice_base_kernel(Geom g, int64_t nnz, const int32_t *__restrict__ indptr,
                                  int32_t *__restrict__ slice_base) {
  const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t ns = g.num_slices();
  if (s > ns) return;
  const int64_t i = s < ns ? g.slice_begin(s) : g.n_items;
  slice_base[s] = (int32_t)clamp64(indptr[i], 0, nnz);
}

// Per-slice inverted lists, one workgroup per slice in each kernel:
//  csc_sort_pass_kernel   a stable LSD radix sort of the slice's entries by
//                         column (8-bit digits, one launch per digit). The
//                         first pass reads the CSR in item order and carries
//                         (slice-local item, fl32(v / |item|)); stability keeps
//                         the items ascending within each column, and the last
//                         pass writes the postings in place.
//  dim_runs_kernel        the slice's dim index (sps_internal.h): each run
//                         of equal sorted columns is one list; counted, then
//                         inserted into the slice's hash table.
constexpr int kSortNT = 1024;
constexpr int kSortWaves = kSortNT / 64;

// The slice's entries go through in tiles of kSortNT, in order: within a
// tile each entry's place is its digit's running base, plus the counts of
// the digit in the waves before its own, plus its rank among the lanes of
// its wave holding the same digit.
template <bool FIRST>
__global__ __launch_bounds__(kSortNT) void csc_sort_pass_kernel(
    Geom g, const int32_t *__restrict__ flags, const int32_t *__restrict__ indptr,
    const int32_t *__restrict__ indices, const float *__restrict__ values,
    const double *__restrict__ norm64, const int32_t *__restrict__ slice_base,
    const int32_t *__restrict__ src_key, const uint2 *__restrict__ src_pay,
    int32_t *__restrict__ dst_key, uint2 *__restrict__ dst_pay, int shift) {
  __shared__ uint32_t s_hist[256];             // digit counts, then running bases
  __shared__ uint32_t s_cnt[kSortWaves][256];  // per-wave digit counts of a tile
  __shared__ int32_t s_ptr[kSliceMax + 1];     // first pass: item starts in the slice
  __shared__ int32_t s_ws[kSortWaves];
  if (flags[0] != 0) return;
  const int64_t sl = blockIdx.x;
  const int64_t b = slice_base[sl];
  const int64_t n = slice_base[sl + 1] - b;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int64_t i0 = g.slice_begin(sl);
  int32_t nitems = 0;
  if (FIRST) {
    nitems = (int32_t)(g.slice_end(sl) - i0);
    for (int k = t; k <= nitems; k += kSortNT) s_ptr[k] = (int32_t)(indptr[i0 + k] - b);
  }
  const int32_t *kin = FIRST ? indices + b : src_key + b;
  if (t < 256) s_hist[t] = 0u;
  __syncthreads();
  // (four tiles' keys in flight at a time)
  for (int64_t i = t; i < n; i += 4 * kSortNT) {
    uint32_t kk[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) kk[u] = i + u * kSortNT < n ? (uint32_t)kin[i + u * kSortNT] : 0u;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i + u * kSortNT < n) atomicAdd(&s_hist[(kk[u] >> shift) & 255u], 1u);
  }
  __syncthreads();
  {
    const int32_t v = t < 256 ? (int32_t)s_hist[t] : 0;
    int32_t tot;
    const int32_t incl = block_incl_scan_1b<kSortNT>(v, s_ws, &tot);
    if (t < 256) s_hist[t] = (uint32_t)(incl - v);
  }
  const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
  uint32_t *cflat = &s_cnt[0][0];
  // the next tile's key and value (or payload) are loaded during this tile
  int32_t nkey = 0;
  uint2 npay = make_uint2(0u, 0u);
  float nval = 0.0f;
  if (t < n) {
    nkey = kin[t];
    if (FIRST) nval = values[b + t];
    else npay = src_pay[b + t];
  }
  for (int64_t base = 0; base < n; base += kSortNT) {
    const int64_t i = base + t;
    const bool valid = i < n;
    int32_t key = 0;
    uint2 pay = make_uint2(0u, 0u);
    const int32_t ckey = nkey;
    const uint2 cpay = npay;
    const float cval = nval;
    if (i + kSortNT < n) {
      nkey = kin[i + kSortNT];
      if (FIRST) nval = values[b + i + kSortNT];
      else npay = src_pay[b + i + kSortNT];
    }
    if (valid) {
      key = ckey;
      if (FIRST) {
        // the item of entry i: the last item starting at or before it
        int lo = 0, hi = nitems;
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (s_ptr[mid] <= i) lo = mid;
          else hi = mid;
        }
        const double nrm = norm64[i0 + lo];
        const float w = nrm > 0.0 ? (float)((double)cval / nrm) : 0.0f;
        pay = make_uint2((uint32_t)lo, __float_as_uint(w));
      } else {
        pay = cpay;
      }
    }
    const uint32_t digit = ((uint32_t)key >> shift) & 255u;
    // the lanes holding the same digit (stable rank = those below this lane)
    uint64_t m = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const bool x = (digit >> bit) & 1u;
      const uint64_t bb = __ballot(x);
      m &= x ? bb : ~bb;
    }
    for (int k = t; k < kSortWaves * 256; k += kSortNT) cflat[k] = 0u;
    __syncthreads();
    if (valid && (m & lt) == 0) s_cnt[wv][digit] = (uint32_t)__popcll(m);
    __syncthreads();
    if (t < 256) {
      uint32_t run = s_hist[t];
      for (int w = 0; w < kSortWaves; ++w) {
        const uint32_t c = s_cnt[w][t];
        s_cnt[w][t] = run;
        run += c;
      }
      s_hist[t] = run;
    }
    __syncthreads();
    if (valid) {
      const int64_t dst = b + s_cnt[wv][digit] + __popcll(m & lt);
      dst_key[dst] = key;
      dst_pay[dst] = pay;
    }
    __syncthreads();  // this tile's offsets are read before the next tile clears them
  }
}

// The slice's dim index (see sps_internal.h) from its sorted columns, one
// workgroup per slice over the sorted keys. An entry ends a run (one dim's
// list) when the next key differs or the slice ends; the run starts at the
// latest entry at or before it whose previous key differs: a running
// maximum, within a lane's four keys and then across the wave (DPP), carried
// from step to step of the wave's own share of the keys.
//  COUNT   distinct dims -> info[s].w; with gdf, every list of at least hmin
//          entries adds its length to gdf[(s % kGdfStripes) * dim + d]
//          (heavy-dim document frequency, summed over the copies later)
//  BUILD   the slice's table, kBuildBuckets buckets at a time in LDS: each
//          sweep over the runs inserts those whose home bucket lies in the
//          range (linear probing in LDS, no global atomics), then the range
//          is written out whole, empty slots included (so the table needs no
//          clearing). A run whose probe would leave the range is deferred and
//          inserted after the last range, by atomic compare-and-swap in the
//          written table from its home bucket: every slot it passes is full
//          by then, so it lands where a plain linear-probing insert would
//          have been allowed to put it, and a lookup from its home finds it.
// A structural fault leaves every slice with no lists.
constexpr int kRunNT = 1024;
constexpr int kBuildBuckets = 8192;  // 128 KiB of 16-byte buckets in LDS per range
constexpr int kDeferCap = 512;       // deferred runs kept in LDS per slice

// The build's deferred-run capacity: kDeferCap, or less when SPS_DIM_DEFER_CAP
// asks (a test hook: 0 sends every deferred run through the fallback sweep).
static int32_t dim_defer_cap() {
  int32_t cap = kDeferCap;
  if (const char *ev = getenv("SPS_DIM_DEFER_CAP")) {
    const long v = atol(ev);
    if (v >= 0 && v < cap) cap = (int32_t)v;
  }
  return cap;
}
enum { kRunsCount = 0, kRunsBuild = 1 };
template <int MODE>
__global__ __launch_bounds__(kRunNT) void dim_runs_kernel(const int32_t *__restrict__ flags,
                                                          const int32_t *__restrict__ slice_base,
                                                          const int32_t *__restrict__ keys,
                                                          int4 *__restrict__ info,
                                                          uint4 *__restrict__ tab,
                                                          int32_t *__restrict__ gdf, int32_t hmin,
                                                          int64_t dim, int32_t defer_cap,
                                                          int32_t *__restrict__ ldim,
                                                          uint2 *__restrict__ lval) {
  constexpr bool BUILD = MODE == kRunsBuild;
  constexpr int NW = kRunNT / 64;
  constexpr unsigned long long kEmpty64 = ~0ull;
  static_assert(kDimEmpty == 0xFFFFFFFFu, "an empty slot is all ones");
  __shared__ int32_t s_cnt;
  __shared__ unsigned long long s_tab[BUILD ? 2 * kBuildBuckets : 1];
  __shared__ uint4 s_def[BUILD ? kDeferCap : 1];  // (first word, second word) of deferred runs
  __shared__ int32_t s_ndef, s_nlist;
  const int64_t sl = blockIdx.x;
  const bool fault = flags[0] != 0;
  const int64_t b = fault ? 0 : slice_base[sl];
  const int64_t n = fault ? 0 : slice_base[sl + 1] - b;
  const int32_t *ks = keys + b;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  int32_t *const gdf_s = gdf == nullptr ? nullptr : gdf + (sl % kGdfStripes) * dim;
  int4 inf = make_int4(0, 1, 0, 0);
  if (BUILD) inf = info[sl];
  if (t == 0) s_cnt = s_ndef = 0;
  __syncthreads();
  // Each wave takes its own contiguous share of the sorted keys (whole steps
  // of 256, four consecutive keys per lane), with no barrier between the
  // waves: a run is reported by the wave holding its last entry, its start
  // found from the run open at the share's first entry (searched backwards, a
  // run being at most one entry per item). visit(dim, start, length) is called
  // once per run.
  constexpr int KPL = 4;  // keys per lane and step
  const int64_t share = ((n + NW - 1) / NW + 64 * KPL - 1) / (64 * KPL) * (64 * KPL);
  const int64_t lo = wv * share, hi = lo + share < n ? lo + share : n;
  auto sweep = [&](auto &&visit) {
    int32_t carry = 0;  // 1 + start of the run open at the current step's first entry
    if (lo < hi && lo > 0) {
      const int32_t k0 = ks[lo];
      int64_t st = lo;
      for (int64_t j = lo - 1; j >= 0; j -= 64) {  // (uniform: ballots decide)
        const int64_t idx = j - lane;
        const bool diff = idx < 0 || ks[idx] != k0;
        const uint64_t m = __ballot(diff);
        if (m != 0ull) {
          st = j - __builtin_ctzll(m) + 1;
          break;
        }
        st = j - 63;
      }
      carry = (int32_t)st + 1;
    }
    for (int64_t base = lo; base < hi; base += 64 * KPL) {
      const int64_t j0 = base + KPL * lane;
      int32_t k[KPL];
#pragma unroll
      for (int u = 0; u < KPL; ++u) k[u] = j0 + u < n ? ks[j0 + u] : -1;  // (-1: no dim)
      // the keys before and after the lane's four (the neighbouring lanes'; the
      // step's ends from memory)
      const int32_t kb = base > 0 ? ks[base - 1] : -1;
      const int32_t ka = base + 64 * KPL < n ? ks[base + 64 * KPL] : -1;
      int32_t prev = __builtin_amdgcn_update_dpp(0, k[KPL - 1], 0x138, 0xf, 0xf, false);  // wave_shr:1
      int32_t next = __builtin_amdgcn_update_dpp(0, k[0], 0x130, 0xf, 0xf, false);  // wave_shl:1
      if (lane == 0) prev = kb;
      if (lane == 63) next = ka;
      bool last[KPL];
      int32_t lm[KPL];  // running maximum of 1 + (a run's first entry) within the lane
#pragma unroll
      for (int u = 0; u < KPL; ++u) {
        const int64_t j = j0 + u;
        const bool valid = j < hi;
        const int32_t kp = u == 0 ? prev : k[u - 1];
        const int32_t kn = u == KPL - 1 ? next : k[u + 1];
        const bool first = valid && (j == 0 || kp != k[u]);
        last[u] = valid && (j == n - 1 || kn != k[u]);
        const int32_t f = first ? (int32_t)j + 1 : 0;
        lm[u] = u == 0 ? f : max(lm[u - 1], f);
      }
      const int32_t incl = wave_incl_max_dpp(lm[KPL - 1]);
      const int32_t excl = __builtin_amdgcn_update_dpp(0, incl, 0x138, 0xf, 0xf, false);
      const int32_t c = max(carry, lane == 0 ? 0 : excl);
      carry = max(carry, __builtin_amdgcn_readlane(incl, 63));
#pragma unroll
      for (int u = 0; u < KPL; ++u) {
        if (!last[u]) continue;
        const int32_t st = max(lm[u], c) - 1;
        visit(k[u], st, (int32_t)(j0 + u) - st + 1);
      }
    }
  };
  if (!BUILD) {
    int32_t mine = 0;  // runs ending in this wave's share
    sweep([&](int32_t kk, int32_t st, int32_t len) {
      ++mine;
      if (gdf_s != nullptr && len >= hmin) atomicAdd(&gdf_s[kk], len);
    });
    mine = wave_sum(mine);
    if (lane == 0 && mine != 0) atomicAdd(&s_cnt, mine);
    __syncthreads();
    if (t == 0) info[sl] = make_int4(0, 0, 0, s_cnt);
    return;
  }
  // BUILD. A slot pair per bucket: narrow tables hold two runs per bucket,
  // (dim | (start | (length - 1) << kStartBits) << 32) each; wide tables one,
  // (dim | start << 32) then (dim | length << 32).
  const uint32_t nb = (uint32_t)inf.y;
  const bool wide = inf.z != 0;
  uint4 *const gtab = tab + inf.x;
  auto words = [&](int32_t kk, int32_t st, int32_t len, unsigned long long &w0,
                   unsigned long long &w1) {
    if (wide) {
      w0 = (uint32_t)kk | ((unsigned long long)(uint32_t)st << 32);
      w1 = (uint32_t)kk | ((unsigned long long)(uint32_t)len << 32);
    } else {
      // a list is at most one entry per item of the slice (canonical CSR)
      const uint32_t lm1 = (uint32_t)(len < kSliceMax ? len : kSliceMax) - 1u;
      w0 = w1 = (uint32_t)kk | ((unsigned long long)((uint32_t)st | (lm1 << kStartBits)) << 32);
    }
  };
  // into the global table from the run's home bucket on: the first free
  // slot, unless a slot on the way already holds the dim (only atomics touch
  // the table here, so no cached copy of it is read)
  auto insert_global = [&](uint32_t bk, unsigned long long w0, unsigned long long w1) {
    unsigned long long *t64 = reinterpret_cast<unsigned long long *>(gtab);
    const uint32_t kk = (uint32_t)w0;
    for (uint32_t tries = 0; tries < nb; ++tries) {
      unsigned long long *slot = t64 + 2 * (int64_t)bk;
      unsigned long long old = atomicCAS(slot, kEmpty64, w0);
      if (old == kEmpty64) {
        if (wide) slot[1] = w1;
        return;
      }
      if ((uint32_t)old == kk) return;
      if (!wide) {
        old = atomicCAS(slot + 1, kEmpty64, w0);
        if (old == kEmpty64 || (uint32_t)old == kk) return;
      }
      bk = bk + 1 == nb ? 0u : bk + 1;
    }
  };
  // The runs whose home bucket lies past the current range go onto a list (the
  // slice's own span of the free sort buffers, at most one run per entry),
  // which the next range reads instead of sweeping the keys again; it
  // rewrites the list in place with the runs still ahead (never past the
  // entries it has read).
  int32_t *const ld = ldim + b;
  uint2 *const lv = lval + b;
  int32_t nlist = 0;  // runs on the list (uniform: read after a barrier)
  for (uint32_t p0 = 0; p0 < nb; p0 += kBuildBuckets) {
    const uint32_t p1 = nb - p0 < (uint32_t)kBuildBuckets ? nb : p0 + kBuildBuckets;
    for (uint32_t i = t; i < 2 * (p1 - p0); i += kRunNT) s_tab[i] = kEmpty64;
    if (t == 0) s_nlist = 0;
    __syncthreads();
    // a run whose home is in [p0, p1) into the range, else onto the list
    auto place = [&](int32_t kk, int32_t st, int32_t len) {
      const uint32_t home = dim_bucket((uint32_t)kk, nb);
      if (home >= p1) {
        const int i = atomicAdd(&s_nlist, 1);
        ld[i] = kk;
        lv[i] = make_uint2((uint32_t)st, (uint32_t)len);
        return;
      }
      unsigned long long w0, w1;
      words(kk, st, len, w0, w1);
      for (uint32_t bk = home; bk < p1; ++bk) {
        unsigned long long *slot = s_tab + 2 * (bk - p0);
        if (wide) {
          if (atomicCAS(slot, kEmpty64, w0) == kEmpty64) {
            slot[1] = w1;
            return;
          }
        } else {
          if (atomicCAS(slot, kEmpty64, w0) == kEmpty64) return;
          if (atomicCAS(slot + 1, kEmpty64, w0) == kEmpty64) return;
        }
      }
      // the probe would leave the range: defer
      const int i = atomicAdd(&s_ndef, 1);
      if (i < defer_cap)
        s_def[i] = make_uint4((uint32_t)w0, (uint32_t)(w0 >> 32), (uint32_t)w1,
                              (uint32_t)(w1 >> 32));
    };
    if (p0 == 0) {
      sweep(place);
    } else {
      for (int32_t cb = 0; cb < nlist; cb += kRunNT) {
        const int32_t i = cb + t;
        int32_t kk = 0;
        uint2 v = make_uint2(0u, 0u);
        if (i < nlist) {
          kk = ld[i];
          v = lv[i];
        }
        __syncthreads();  // (this block of the list is read before any of it is rewritten)
        if (i < nlist) place(kk, (int32_t)v.x, (int32_t)v.y);
      }
    }
    __syncthreads();
    nlist = s_nlist;
    const uint4 *st4 = reinterpret_cast<const uint4 *>(s_tab);
    for (uint32_t i = t; i < p1 - p0; i += kRunNT) gtab[p0 + i] = st4[i];
    __syncthreads();  // (the range is read before the next one clears it)
  }
  // the deferred runs, into the written table (its stores are complete: the
  // barrier above waited for them)
  const int nd = s_ndef;  // (uniform: read after the last barrier)
  for (int i = t; i < (nd < defer_cap ? nd : defer_cap); i += kRunNT) {
    const uint4 d = s_def[i];
    const unsigned long long w0 = d.x | ((unsigned long long)d.y << 32);
    const unsigned long long w1 = d.z | ((unsigned long long)d.w << 32);
    insert_global(dim_bucket(d.x, nb), w0, w1);
  }
  if (nd <= defer_cap) return;
  // More deferred runs than s_def holds (a table far from its usual fill):
  // every run not yet in the table goes in by the same global insert.
  __syncthreads();
  sweep([&](int32_t kk, int32_t st, int32_t len) {
    unsigned long long w0, w1;
    words(kk, st, len, w0, w1);
    insert_global(dim_bucket((uint32_t)kk, nb), w0, w1);
  });
}

// gdf[d] += gdf[s * dim + d] for the other copies s
__global__ void gdf_fold_kernel(int64_t dim, int32_t *__restrict__ gdf) {
  for (int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; d < dim;
       d += (int64_t)gridDim.x * blockDim.x) {
    int32_t v = gdf[d];
#pragma unroll
    for (int s = 1; s < kGdfStripes; ++s) v += gdf[s * dim + d];
    gdf[d] = v;
  }
}

// Bucket ranges of the slices' tables (one workgroup): nb = max(1, 2 distinct),
// first bucket = the sum over earlier slices; info[ns].x = total buckets.
__global__ __launch_bounds__(1024) void dim_layout_kernel(int64_t ns,
                                                          const int32_t *__restrict__ slice_base,
                                                          int4 *__restrict__ info) {
  __shared__ int32_t ws[16];
  int32_t carry = 0;
  for (int64_t base = 0; base < ns; base += 1024) {
    const int64_t s = base + threadIdx.x;
    int4 x = make_int4(0, 0, 0, 0);
    int32_t nb = 0;
    if (s < ns) {
      x = info[s];
      nb = x.w > 0 ? kBucketsPerDim * x.w : 1;
    }
    int32_t tot;
    const int32_t incl = block_incl_scan<1024>(nb, ws, &tot);
    if (s < ns) {
      const int64_t nnz_s = (int64_t)slice_base[s + 1] - slice_base[s];
      info[s] = make_int4(carry + incl - nb, nb, nnz_s > kNarrowMaxNnz ? 1 : 0, x.w);
    }
    carry += tot;
  }
  if (threadIdx.x == 0) info[ns] = make_int4(carry, 0, 0, 0);
}

// col_ptr of one slice from its index (for verification and tools): dims
// with a list take their start, the others (and the end) the slice's entry
// count, then a suffix minimum gives every dim the start of the next list.
__global__ void expand_starts_kernel(int64_t dim, const int4 *__restrict__ dinfo,
                                     const uint4 *__restrict__ dtab,
                                     const int32_t *__restrict__ slice_base, int64_t slice,
                                     int32_t *__restrict__ cp) {
  const int4 inf = dinfo[slice];
  const int32_t nnz_s = slice_base[slice + 1] - slice_base[slice];
  for (int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; d <= dim;
       d += (int64_t)gridDim.x * blockDim.x) {
    int32_t st = nnz_s, len = 0;
    if (d < dim && !dim_lookup(dtab, inf, (uint32_t)d, st, len)) st = nnz_s;
    cp[d] = st;
  }
}

__global__ __launch_bounds__(1024) void suffix_min_kernel(int64_t n, int32_t *__restrict__ a) {
  __shared__ int32_t ws[16];
  int32_t carry = 0x7fffffff;
  for (int64_t top = n; top > 0; top -= 1024) {
    // element top - 1 - t, so that lane order runs from the end
    const int64_t j = top - 1 - threadIdx.x;
    const int32_t v = j >= 0 ? a[j] : 0x7fffffff;
    // inclusive running minimum = -(running maximum of -v), via biased values
    const uint32_t biased = 0x7fffffffu - (uint32_t)v;  // v >= 0: fits, and order reverses
    int32_t m = wave_incl_max_dpp((int32_t)biased);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    if (lane == 63) ws[wv] = m;
    __syncthreads();
    int32_t tmax = 0;
    for (int w = 0; w < 16; ++w) {
      if (w < wv) m = max(m, ws[w]);
      tmax = max(tmax, ws[w]);
    }
    __syncthreads();
    const int32_t runmin = 0x7fffffff - m;
    if (j >= 0) a[j] = min(runmin, carry);
    carry = min(carry, 0x7fffffff - tmax);
  }
}

// *status |= 1 where a list's start plus its length is not the next entry of col_ptr
__global__ void expand_check_kernel(int64_t dim, const int4 *__restrict__ dinfo,
                                    const uint4 *__restrict__ dtab, int64_t slice,
                                    const int32_t *__restrict__ cp, int32_t *status) {
  const int4 inf = dinfo[slice];
  for (int64_t d = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; d < dim;
       d += (int64_t)gridDim.x * blockDim.x) {
    int32_t st = 0, len = 0;
    if (dim_lookup(dtab, inf, (uint32_t)d, st, len) && (cp[d] != st || cp[d + 1] != st + len))
      atomicOr(status, 1);
  }
}

hipError_t launch_expand_col_ptr(int64_t dim, const int4 *dinfo, const uint4 *dtab,
                                 const int32_t *slice_base, int64_t slice, int32_t *col_ptr,
                                 int32_t *status, hipStream_t s) {
  int64_t blocks = (dim + 1 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(expand_starts_kernel, dim3((unsigned)blocks), dim3(256), 0, s, dim, dinfo,
                     dtab, slice_base, slice, col_ptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(suffix_min_kernel, dim3(1), dim3(1024), 0, s, dim + 1, col_ptr);
  if ((e = hipGetLastError()) != hipSuccess || status == nullptr) return e;
  hipLaunchKernelGGL(expand_check_kernel, dim3((unsigned)blocks), dim3(256), 0, s, dim, dinfo,
                     dtab, slice, col_ptr, status);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Heavy dims. A few dims are held by most items (term ids follow a steep
// rank law; the page notes ids cluster in a dictionary prefix, §3.2). For
// those a posting list covers most of a slice, and a dense row of the slice
// ("slab": value per item, 0 where absent) lets the score kernel use
// matrix-core FMAs instead of per-entry scatter. Selection: dims whose
// document frequency is at least n_items / kHeavyFracInv, the kHeavyMax most
// frequent (ties: lower dim), listed in ascending dim order. The choice only
// affects speed; both paths compute the same sums.
// ---------------------------------------------------------------------------

constexpr int kCandCap = 2048;
static_assert(kHeavySelInts == 33 + 2 * kCandCap, "heavy-dim selection scratch layout");

// Heavy-dim choice in three launches over gdf (hsel: 32 level counts, the
// candidate count, kCandCap candidate dims, kCandCap their frequencies; the
// first 33 zeroed). Level k counts the dims with gdf in [tglob * 2^k,
// tglob * 2^(k+1)); the candidates are the dims at or above the lowest level
// whose tail still fits kCandCap, and the heavy dims are the `cap` most
// frequent candidates (ties to the lower dim), stored ascending.
__global__ __launch_bounds__(256) void heavy_level_kernel(const int32_t *__restrict__ gdf,
                                                         int64_t dim, int32_t tglob,
                                                         const int32_t *__restrict__ flags,
                                                         int32_t *__restrict__ hsel) {
  __shared__ int32_t s_lvl[32];
  const int t = threadIdx.x;
  if (flags[0] != 0 || tglob <= 0) return;
  if (t < 32) s_lvl[t] = 0;
  __syncthreads();
  for (int64_t d = (int64_t)blockIdx.x * 256 + t; d < dim; d += (int64_t)gridDim.x * 256) {
    const int32_t v = gdf[d];
    if (v >= tglob) atomicAdd(&s_lvl[31 - __clz((unsigned)(v / tglob))], 1);
  }
  __syncthreads();
  if (t < 32 && s_lvl[t] != 0) atomicAdd(&hsel[t], s_lvl[t]);
}

__device__ __forceinline__ int heavy_level(const int32_t *hsel) {
  int above = 0, level = 31;
  for (int k = 31; k >= 0; --k) {  // lowest level whose tail still fits the candidate cap
    if (above + hsel[k] > kCandCap) break;
    above += hsel[k];
    level = k;
  }
  return level;
}

__global__ __launch_bounds__(256) void heavy_collect_kernel(const int32_t *__restrict__ gdf,
                                                           int64_t dim, int32_t tglob,
                                                           const int32_t *__restrict__ flags,
                                                           int32_t *__restrict__ hsel) {
  __shared__ int32_t s_level;
  const int t = threadIdx.x;
  if (flags[0] != 0 || tglob <= 0) return;
  if (t == 0) s_level = heavy_level(hsel);
  __syncthreads();
  const int64_t thr = (int64_t)tglob << s_level;
  int32_t *cd = hsel + 33, *cv = hsel + 33 + kCandCap;
  for (int64_t d = (int64_t)blockIdx.x * 256 + t; d < dim; d += (int64_t)gridDim.x * 256) {
    const int32_t v = gdf[d];
    if ((int64_t)v >= thr) {
      const int i = atomicAdd(&hsel[32], 1);
      if (i < kCandCap) {
        cd[i] = (int32_t)d;
        cv[i] = v;
      }
    }
  }
}

// How many blocks of kHeavyBlock dims: the first always; block b (the
// candidates of frequency rank 32 b .. 32 b + 31) while the sum over its dims
// of (df / n_items)^2 exceeds `gain`. That sum is what the block takes off
// the sparse walk per score, in (query entry, posting) products, if queries
// hold each dim about as often as items do; a block on the matrix cores
// costs about as much as `gain` such products per score.
__global__ __launch_bounds__(1024) void heavy_rank_kernel(int32_t cap, float gain,
                                                         int64_t n_items,
                                                         const int32_t *__restrict__ flags,
                                                         const int32_t *__restrict__ hsel,
                                                         int32_t *__restrict__ heavy) {
  constexpr int NT = 1024;
  __shared__ int32_t s_cd[kCandCap], s_cv[kCandCap];
  __shared__ int16_t s_rank[kCandCap];
  __shared__ unsigned long long s_bsum[kHeavyBlocksMax];
  __shared__ int32_t s_count;
  const int t = threadIdx.x;
  if (flags[0] != 0 || cap <= 0) {
    if (t == 0) heavy[kHeavyMax] = 0;
    return;
  }
  const int n = hsel[32] < kCandCap ? hsel[32] : kCandCap;
  for (int i = t; i < n; i += NT) {
    s_cd[i] = hsel[33 + i];
    s_cv[i] = hsel[33 + kCandCap + i];
  }
  if (t < kHeavyBlocksMax) s_bsum[t] = 0ull;
  __syncthreads();
  for (int i = t; i < n; i += NT) {
    int rank = 0;
    const int32_t vi = s_cv[i], di = s_cd[i];
    for (int j = 0; j < n; ++j) {
      const int32_t vj = s_cv[j], dj = s_cd[j];
      rank += (vj > vi || (vj == vi && dj < di)) ? 1 : 0;
    }
    s_rank[i] = (int16_t)rank;
    if (rank < cap) atomicAdd(&s_bsum[rank / kHeavyBlock], (unsigned long long)vi * (uint64_t)vi);
  }
  __syncthreads();
  if (t == 0) {
    const int lim = n < cap ? n : cap;
    const double nn = (double)n_items * (double)n_items;
    int nb = 1;
    while (nb < heavy_blocks(lim) && (double)s_bsum[nb] > (double)gain * nn) ++nb;
    s_count = lim < nb * kHeavyBlock ? lim : nb * kHeavyBlock;
  }
  __syncthreads();
  const int count = s_count;
  for (int i = t; i < n; i += NT) {
    if (s_rank[i] >= count) continue;
    int pos = 0;
    for (int j = 0; j < n; ++j) pos += (s_rank[j] < count && s_cd[j] < s_cd[i]) ? 1 : 0;
    heavy[pos] = s_cd[i];
  }
  if (t == 0) heavy[kHeavyMax] = count;
}

// slab of slice c (one workgroup per slice), block by block of kHeavyBlock
// heavy dims in use: the block's tiles are assembled in LDS (zeroed, then
// each of its dims' lists written in as split-fp16 values; wave w takes the
// block's dims w, w + 16, ...) and written out whole. Blocks past the ones in
// use are never read.
constexpr int kSlabNT = 1024;
__global__ __launch_bounds__(kSlabNT) void slab_scatter_kernel(
    int32_t pitch, int64_t bstride, const int32_t *__restrict__ flags,
    const int32_t *__restrict__ heavy,
    const int4 *__restrict__ dinfo, const uint4 *__restrict__ dtab,
    const int32_t *__restrict__ slice_base, const uint2 *__restrict__ post,
    uint16_t *__restrict__ slab) {
  constexpr int NW = kSlabNT / 64;
  constexpr int kBlockHalves = kSliceMax * kHeavyRec;  // one block of a whole slice
  __shared__ uint4 s_blk[kBlockHalves * 2 / 16];
  uint16_t *const sh = reinterpret_cast<uint16_t *>(s_blk);
  const int64_t c = blockIdx.x;
  if (flags[0] != 0) return;
  const int count = heavy[kHeavyMax];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int64_t base = slice_base[c];
  const int32_t snnz = slice_base[c + 1] - slice_base[c];
  const int words = pitch * kHeavyRec * 2 / 16;  // 16-byte words of the slice's block
  for (int hb = 0; hb < heavy_blocks(count); ++hb) {
    for (int i = t; i < words; i += kSlabNT) s_blk[i] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    const int hend = count < (hb + 1) * kHeavyBlock ? count : (hb + 1) * kHeavyBlock;
    for (int h = hb * kHeavyBlock + wv; h < hend; h += NW) {
      int32_t b = 0, len = 0;
      if (!dim_lookup(dtab, dinfo[c], (uint32_t)heavy[h], b, len)) continue;
      const int32_t e = (int32_t)clamp64((int64_t)b + len, 0, snnz);
      // (four postings in flight per lane)
      for (int32_t k0 = b + lane; k0 < e; k0 += 4 * 64) {
        uint2 pe[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          pe[u] = k0 + 64 * u < e ? post[base + k0 + 64 * u] : make_uint2(0xFFFFFFFFu, 0u);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (pe[u].x < (uint32_t)pitch) {
            uint16_t hi, lo;
            split_fp16(__uint_as_float(pe[u].y), hi, lo);
            uint16_t *tile = sh + (pe[u].x >> 4) * kTileHalves;
            tile[heavy_tile_index(pe[u].x, h, 0)] = hi;
            tile[heavy_tile_index(pe[u].x, h, 1)] = lo;
          }
        }
      }
    }
    __syncthreads();
    uint4 *dst = reinterpret_cast<uint4 *>(slab + hb * bstride + c * (int64_t)pitch * kHeavyRec);
    for (int i = t; i < words; i += kSlabNT) dst[i] = s_blk[i];
    __syncthreads();  // (read out before the next block clears it)
  }
}

hipError_t launch_prepare_items(const ItemsDev &d, hipStream_t s) {
  hipError_t e;
  const Geom &g = d.g;
  const int64_t ns = g.num_slices();
  e = launch_csr_check(g.n_items, d.dim, d.nnz, d.indptr, d.indices, d.values, 0, d.flags, s);
  if (e != hipSuccess) return e;
  e = launch_row_norms(g.n_items, d.nnz, d.indptr, d.values, d.flags, d.inv_norm, d.norm64, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(slice_base_kernel, dim3((unsigned)((ns + 1 + 255) / 256)), dim3(256), 0, s,
                     g, d.nnz, d.indptr, d.slice_base);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  e = launch_fill_i32(d.heavy, kHeavyMax + 1, 0, s);
  if (e != hipSuccess) return e;
  e = launch_fill_i32(reinterpret_cast<int32_t *>(d.post + d.nnz), 2 * kPostPad, 0, s);
  if (e != hipSuccess) return e;
  if (g.n_items == 0) return hipSuccess;
  if (d.dense) {
    e = launch_fill_i32(d.gdf, kGdfStripes * d.dim, 0, s);
    if (e != hipSuccess) return e;
  }
  // radix passes: 8-bit digits of the largest column, at least one (the
  // first pass also builds the payload); the last one writes the postings
  int bits = 0;
  while (bits < 31 && (d.dim - 1) >> bits > 0) ++bits;
  const int passes = bits > 8 ? (bits + 7) / 8 : 1;
  for (int p = 0; p < passes; ++p) {
    int32_t *kd = ((passes - 1 - p) & 1) ? d.skey[1] : d.skey[0];
    uint2 *pd = ((passes - 1 - p) & 1) ? d.spay : d.post;
    const int32_t *ks = ((passes - p) & 1) ? d.skey[1] : d.skey[0];
    const uint2 *ps = ((passes - p) & 1) ? d.spay : d.post;
    if (p == 0)
      hipLaunchKernelGGL(csc_sort_pass_kernel<true>, dim3((unsigned)ns), dim3(kSortNT), 0, s, g,
                         d.flags, d.indptr, d.indices, d.values, d.norm64, d.slice_base, nullptr,
                         nullptr, kd, pd, 0);
    else
      hipLaunchKernelGGL(csc_sort_pass_kernel<false>, dim3((unsigned)ns), dim3(kSortNT), 0, s, g,
                         d.flags, d.indptr, d.indices, d.values, d.norm64, d.slice_base, ks, ps,
                         kd, pd, 8 * p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // the dim index: count the lists, lay out the tables, build them
  const int32_t hmin = g.S / (2 * kHeavyFracInv) > 2 ? g.S / (2 * kHeavyFracInv) : 2;
  hipLaunchKernelGGL(dim_runs_kernel<kRunsCount>, dim3((unsigned)ns), dim3(kRunNT), 0, s, d.flags,
                     d.slice_base, d.skey[0], d.dinfo, d.dtab, d.dense ? d.gdf : nullptr, hmin,
                     d.dim, 0, nullptr, nullptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(dim_layout_kernel, dim3(1), dim3(1024), 0, s, ns, d.slice_base, d.dinfo);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(dim_runs_kernel<kRunsBuild>, dim3((unsigned)ns), dim3(kRunNT), 0, s, d.flags,
                     d.slice_base, d.skey[0], d.dinfo, d.dtab, nullptr, 0, d.dim,
                     dim_defer_cap(), d.skey[1], d.spay);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (!d.dense) return hipSuccess;
  const int64_t tg64 = (g.n_items + kHeavyFracInv - 1) / kHeavyFracInv;
  const int32_t tglob = (int32_t)(tg64 > 2 ? tg64 : 2);
  e = launch_fill_i32(d.hsel, 33, 0, s);
  if (e != hipSuccess) return e;
  int64_t hblocks = (d.dim + 255) / 256;
  if (hblocks > 1024) hblocks = 1024;
  hipLaunchKernelGGL(gdf_fold_kernel, dim3((unsigned)hblocks), dim3(256), 0, s, d.dim, d.gdf);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(heavy_level_kernel, dim3((unsigned)hblocks), dim3(256), 0, s, d.gdf, d.dim,
                     tglob, d.flags, d.hsel);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(heavy_collect_kernel, dim3((unsigned)hblocks), dim3(256), 0, s, d.gdf, d.dim,
                     tglob, d.flags, d.hsel);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(heavy_rank_kernel, dim3(1), dim3(1024), 0, s, d.heavy_cap, d.heavy_gain,
                     g.n_items, d.flags, d.hsel, d.heavy);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (d.heavy_cap <= 0) return hipSuccess;
  const int32_t pitch = slab_pitch(g.S);
  hipLaunchKernelGGL(slab_scatter_kernel, dim3((unsigned)ns), dim3(kSlabNT), 0, s, pitch,
                     d.slab_bstride, d.flags, d.heavy, d.dinfo, d.dtab, d.slice_base, d.post,
                     d.slab);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Reduced-precision variant: 4-byte postings, the slice-local item id (< 2^16)
// in the low half and fp16(256 w) in the high half (256 w is exact in fp32;
// the scale keeps normalised values down to 2^-22 in fp16's normal range).
// ---------------------------------------------------------------------------

__global__ void pack_half_kernel(const uint2 *__restrict__ post, int64_t nnz,
                                 uint32_t *__restrict__ post4) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nnz) {
    const uint2 p = post[i];
    const _Float16 h = (_Float16)(__uint_as_float(p.y) * kHeavyScale);
    post4[i] = (p.x & 0xFFFFu) | ((uint32_t)__builtin_bit_cast(uint16_t, h) << 16);
  } else if (i < nnz + kPostPad4) {
    post4[i] = 0u;
  }
}

hipError_t launch_pack_half(const uint2 *post, int64_t nnz, uint32_t *post4, hipStream_t s) {
  const int64_t n = nnz + kPostPad4;
  hipLaunchKernelGGL(pack_half_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, post,
                     nnz, post4);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Queries. Each row is normalised by its float64 norm (§5.2) and rounded
// once to fp32: qn = fl32(q_d / |q|). Heavy dims (dense path) go to the
// row's split-fp16 record in qh (rows padded to a multiple of kRows); the
// other entries form the "light" CSR (same row order) of 12-byte records
// (dim, value, row's position in its group), one load each in the score
// kernel, with values qn * 2^30 (exact: a power of two), the scale of the
// fixed-point accumulators.
// ---------------------------------------------------------------------------

template <bool FILL>
__global__ __launch_bounds__(256) void light_split_kernel(
    int64_t n_rows, const int32_t *__restrict__ indptr, const int32_t *__restrict__ indices,
    const float *__restrict__ values, const double *__restrict__ norm64,
    const int32_t *__restrict__ flags, const int32_t *__restrict__ heavy, int32_t qh_gstride,
    int32_t *__restrict__ lptr, uint3 *__restrict__ lrec, uint16_t *__restrict__ qh) {
  // the heavy list in LDS: each entry's search over it is then a few LDS reads
  // rather than dependent global loads
  __shared__ int32_t s_heavy[kHeavyMax];
  const int m = heavy != nullptr ? heavy[kHeavyMax] : 0;
  for (int i = threadIdx.x; i < m; i += blockDim.x) s_heavy[i] = heavy[i];
  __syncthreads();
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= n_rows) return;
  int64_t b = 0, e = 0;
  if (flags[0] == 0) {
    b = indptr[q];
    e = indptr[q + 1];
  }
  const double n = norm64[q];
  const int rq = (int)(q % kRows);
  int64_t out = FILL ? lptr[q] : 0;
  int32_t count = 0;
  for (int64_t k = b; k < e; ++k) {
    const int32_t d = indices[k];
    const int hs = m > 0 ? heavy_slot(s_heavy, m, d) : -1;
    if (FILL) {
      const float v = (n > 0.0) ? (float)((double)values[k] / n) : 0.0f;
      if (hs >= 0) {
        uint16_t hi, lo;
        split_fp16(v, hi, lo);
        uint16_t *tile = qh + (q / kRows) * qh_gstride + (hs / kHeavyBlock) * kTileHalves;
        tile[heavy_tile_index((int)(q % kRows), hs, 0)] = hi;
        tile[heavy_tile_index((int)(q % kRows), hs, 1)] = lo;
      } else {
        lrec[out] = make_uint3((uint32_t)d, __float_as_uint(v * kFixScale), (uint32_t)rq);
      }
    }
    if (hs < 0) {
      ++out;
      ++count;
    }
  }
  if (!FILL) lptr[q + 1] = count;
}

// Each 16-row group's light records sorted by dim, so that the rows of a
// group that share a dim walk the same posting list in adjacent segments
// (one L1 request serves them). The score kernel's sums do not depend on the
// order of the records; a group of more than kLightSortCap records keeps the
// row order.
constexpr int kLightSortNT = 512;
constexpr int kLightSortCap = 2 * kLightSortNT;
__global__ __launch_bounds__(kLightSortNT) void light_sort_kernel(int64_t n_rows,
                                                                  const int32_t *__restrict__ lptr,
                                                                  uint3 *__restrict__ lrec) {
  __shared__ uint32_t s_key[kLightSortCap];
  __shared__ uint16_t s_idx[kLightSortCap];
  const int64_t g = blockIdx.x;
  const int64_t r1 = (g + 1) * kRows < n_rows ? (g + 1) * kRows : n_rows;
  const int64_t b = lptr[g * kRows], e = lptr[r1];
  const int64_t n = e - b;
  if (n <= 1 || n > kLightSortCap) return;  // uniform per workgroup
  int P = 2;
  while (P < n) P <<= 1;
  const int t = threadIdx.x;
  for (int i = t; i < P; i += kLightSortNT) {
    s_key[i] = i < n ? lrec[b + i].x : 0xFFFFFFFFu;
    s_idx[i] = (uint16_t)i;
  }
  __syncthreads();
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = t; i < P; i += kLightSortNT) {
        const int l = i ^ j;
        if (l > i) {
          const uint32_t ki = s_key[i], kl = s_key[l];
          const bool up = (i & k) == 0;
          if (up ? (ki > kl) : (ki < kl)) {
            s_key[i] = kl;
            s_key[l] = ki;
            const uint16_t x = s_idx[i];
            s_idx[i] = s_idx[l];
            s_idx[l] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  // every record is read before any is written back
  uint3 r[kLightSortCap / kLightSortNT];
#pragma unroll
  for (int m = 0; m < kLightSortCap / kLightSortNT; ++m) {
    const int i = t + m * kLightSortNT;
    if (i < n) r[m] = lrec[b + s_idx[i]];
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < kLightSortCap / kLightSortNT; ++m) {
    const int i = t + m * kLightSortNT;
    if (i < n) lrec[b + i] = r[m];
  }
}

hipError_t launch_prepare_queries(const QueriesDev &d, hipStream_t s) {
  hipError_t e;
  e = launch_csr_check(d.n_rows, d.dim, d.nnz, d.indptr, d.indices, d.values, 0, d.flags, s);
  if (e != hipSuccess) return e;
  e = launch_row_norms(d.n_rows, d.nnz, d.indptr, d.values, d.flags, d.inv_norm, d.norm64, s);
  if (e != hipSuccess) return e;
  e = launch_fill_i32(d.lptr, d.n_rows + 1, 0, s);
  if (e != hipSuccess) return e;
  if (d.n_rows == 0) return hipSuccess;
  if (d.dense) {
    e = launch_fill_i32(reinterpret_cast<int32_t *>(d.qh), (int64_t)d.n_groups * d.qh_gstride / 2,
                        0, s);
    if (e != hipSuccess) return e;
  }
  const int32_t *heavy = d.dense ? d.heavy : nullptr;
  const unsigned blocks = (unsigned)((d.n_rows + 255) / 256);
  hipLaunchKernelGGL(light_split_kernel<false>, dim3(blocks), dim3(256), 0, s, d.n_rows,
                     d.indptr, d.indices, d.values, d.norm64, d.flags, heavy, d.qh_gstride,
                     d.lptr, d.lrec, d.qh);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_scan_inplace(d.lptr, d.n_rows + 1, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(light_split_kernel<true>, dim3(blocks), dim3(256), 0, s, d.n_rows,
                     d.indptr, d.indices, d.values, d.norm64, d.flags, heavy, d.qh_gstride,
                     d.lptr, d.lrec, d.qh);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(light_sort_kernel, dim3((unsigned)d.n_groups), dim3(kLightSortNT), 0, s,
                     d.n_rows, d.lptr, d.lrec);
  return hipGetLastError();
}

}  // namespace sps
