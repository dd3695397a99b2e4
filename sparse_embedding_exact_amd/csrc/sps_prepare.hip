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
//   light_* kernels      query rows split into heavy values and the rest
//
// All kernels are wave64. Device-side guards keep every access inside the
// buffers the host sized, whatever the CSR contents: the prepare calls run
// csr_check_kernel first and every later kernel exits when it found a
// structural fault.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sps_device.h"
#include "sps_internal.h"

namespace sps {

// ---------------------------------------------------------------------------
// small utilities
// ---------------------------------------------------------------------------

__global__ void fill_i32_kernel(int32_t *__restrict__ p, int64_t n, int32_t v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) p[i] = v;
}

hipError_t launch_fill_i32(int32_t *p, int64_t n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

// single-workgroup inclusive scan in place over a[0..n)
template <int NT>
__global__ __launch_bounds__(NT) void scan_inplace_kernel(int32_t *__restrict__ a, int64_t n) {
  __shared__ int32_t ws[NT / 64];
  int32_t carry = 0;
  for (int64_t base = 0; base < n; base += NT) {
    const int64_t j = base + threadIdx.x;
    const int32_t v = j < n ? a[j] : 0;
    int32_t tot;
    const int32_t incl = block_incl_scan<NT>(v, ws, &tot);
    if (j < n) a[j] = carry + incl;
    carry += tot;
  }
}

hipError_t launch_scan_inplace(int32_t *a, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(scan_inplace_kernel<1024>, dim3(1), dim3(1024), 0, s, a, n);
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

// Rows are checked as in a plain loop over each row; a workgroup whose 256
// row pointers are all in order and in range stages the rows' indices (and
// values, for the full check) through LDS in windows, with coalesced loads.
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
// lists occupy that same entry range of row[] / val[], with item ids local to
// the slice.
//
//  1. count   : tickets t = atomicAdd(&cnt[s][d], 1) (arbitrary order)
//  2. scan    : col_ptr[s] = exclusive prefix of cnt[s]; list of dims whose
//               list holds >= 2 entries (compacted, ascending)
//  3. scatter : entry -> position col_ptr[s][d] + t; single-entry lists are
//               final, longer lists go to a temporary area
//  4. fixup   : each longer list is put in ascending item order. Item ids
//               are distinct inside one list, so the rank of an entry is the
//               number of smaller ids: a wave compares ids directly for
//               lists up to 64 entries, a workgroup counts bits of an item
//               bitmap (prefix popcounts) for longer ones.
// The result is the unique CSC with ascending item ids per dim, independent
// of the order the atomics were served in.
// ---------------------------------------------------------------------------

__global__ void slice_base_kernel(Geom g, int64_t nnz, const int32_t *__restrict__ indptr,
                                  int32_t *__restrict__ slice_base) {
  const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t ns = g.num_slices();
  if (s > ns) return;
  const int64_t i = s < ns ? g.slice_begin(s) : g.n_items;
  slice_base[s] = (int32_t)clamp64(indptr[i], 0, nnz);
}

// 16 lanes per item, so that a row's indices are read coalesced.
constexpr int kLanesPerItem = 16;

__global__ __launch_bounds__(256) void csc_count_kernel(Geom g, int64_t dim,
                                                        const int32_t *__restrict__ indptr,
                                                        const int32_t *__restrict__ indices,
                                                        const int32_t *__restrict__ flags,
                                                        int32_t *__restrict__ col_ptr,
                                                        int32_t *__restrict__ ticket) {
  const int64_t gt = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t i = gt / kLanesPerItem;
  const int sub = (int)(gt % kLanesPerItem);
  if (i >= g.n_items || flags[0] != 0) return;
  const int64_t b = indptr[i], e = indptr[i + 1];
  int32_t *cp = col_ptr + g.slice_of(i) * cp_pitch(dim);
  for (int64_t k = b + sub; k < e; k += kLanesPerItem) ticket[k] = atomicAdd(&cp[indices[k]], 1);
}

// One workgroup per slice: exclusive scan of dim+1 counts in place, each
// thread owning 8 consecutive counts of a tile (two 16-byte loads, issued
// for the next tile before this one is scanned and stored); plus
// the compacted list of dims with >= 2 entries. The scan carries (count,
// multi-flag) packed in one 64-bit value: slice nnz < 2^31 keeps the count
// half from carrying into the flag half.
// When gdf is given, every dim holding at least `hmin` entries of the slice
// adds its count to gdf[d] (the document frequency used to pick heavy dims;
// integer atomics, so the totals do not depend on the order of slices).
template <int NT>
__global__ __launch_bounds__(NT) void csc_scan_kernel(int64_t dim,
                                                      const int32_t *__restrict__ flags,
                                                      const int32_t *__restrict__ slice_base,
                                                      int32_t *__restrict__ col_ptr,
                                                      int32_t *__restrict__ mlist,
                                                      int32_t *__restrict__ mcount,
                                                      int32_t *__restrict__ gdf, int32_t hmin) {
  constexpr int PER = 8;
  constexpr int TILE = PER * NT;
  __shared__ int64_t ws[NT / 64];
  const int64_t c = blockIdx.x;
  const int t = threadIdx.x;
  if (flags[0] != 0) {
    if (t == 0) mcount[c] = 0;
    return;
  }
  const int64_t pitch = cp_pitch(dim);  // a multiple of 4: the int4 accesses stay inside
  int4 *cp4 = reinterpret_cast<int4 *>(col_ptr + c * pitch);
  int32_t *ml = mlist + (slice_base[c] / 2 + c);
  const int64_t n = dim + 1;
  int64_t carry = 0;
  // the next tile's counts are loaded while this one is scanned and stored
  int4 x[PER / 4], xn[PER / 4];
  auto load = [&](int64_t base, int4 (&dst)[PER / 4]) {
#pragma unroll
    for (int k = 0; k < PER / 4; ++k) {
      const int64_t j = base + (int64_t)PER * t + 4 * k;
      dst[k] = j < pitch ? cp4[j >> 2] : make_int4(0, 0, 0, 0);
    }
  };
  load(0, x);
  for (int64_t base = 0; base < n; base += TILE) {
    const int64_t j0 = base + (int64_t)PER * t;
    if (base + TILE < n) load(base + TILE, xn);
    int32_t v[PER];
#pragma unroll
    for (int k = 0; k < PER / 4; ++k) {
      const int64_t j = j0 + 4 * k;
      v[4 * k] = j < n ? x[k].x : 0;
      v[4 * k + 1] = j + 1 < n ? x[k].y : 0;
      v[4 * k + 2] = j + 2 < n ? x[k].z : 0;
      v[4 * k + 3] = j + 3 < n ? x[k].w : 0;
    }
    int64_t sum = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      sum += (int64_t)v[k] + ((int64_t)(v[k] >= 2) << 32);
      if (gdf != nullptr && v[k] >= hmin) atomicAdd(&gdf[j0 + k], v[k]);
    }
    int64_t tot;
    const int64_t incl = block_incl_scan<NT>(sum, ws, &tot);
    int64_t ex = carry + incl - sum;
    int32_t o[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      o[k] = (int32_t)(ex & 0xFFFFFFFFll);
      if (v[k] >= 2) ml[ex >> 32] = (int32_t)(j0 + k);
      ex += (int64_t)v[k] + ((int64_t)(v[k] >= 2) << 32);
    }
#pragma unroll
    for (int k = 0; k < PER / 4; ++k) {
      const int64_t j = j0 + 4 * k;
      if (j + 3 < n) {
        cp4[j >> 2] = make_int4(o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]);
      } else {
        int32_t *cp = col_ptr + c * pitch;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (j + u < n) cp[j + u] = o[4 * k + u];
      }
    }
    carry += tot;
#pragma unroll
    for (int k = 0; k < PER / 4; ++k) x[k] = xn[k];
  }
  if (t == 0) mcount[c] = (int32_t)(carry >> 32);
}

__global__ __launch_bounds__(256) void csc_scatter_kernel(
    Geom g, int64_t dim, const int32_t *__restrict__ indptr, const int32_t *__restrict__ indices,
    const float *__restrict__ values, const double *__restrict__ norm64,
    const int32_t *__restrict__ flags, const int32_t *__restrict__ col_ptr,
    const int32_t *__restrict__ slice_base, const int32_t *__restrict__ ticket,
    uint2 *__restrict__ post, uint16_t *__restrict__ trow, float *__restrict__ tval) {
  const int64_t gt = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t i = gt / kLanesPerItem;
  const int sub = (int)(gt % kLanesPerItem);
  if (i >= g.n_items || flags[0] != 0) return;
  const int64_t sl = g.slice_of(i);
  const int32_t *cp = col_ptr + sl * cp_pitch(dim);
  const int64_t base = slice_base[sl];
  const uint16_t local = (uint16_t)(i - g.slice_begin(sl));
  const double n = norm64[i];
  const int64_t b = indptr[i], e = indptr[i + 1];
  for (int64_t k = b + sub; k < e; k += kLanesPerItem) {
    const int32_t d = indices[k];
    const int32_t s = cp[d];
    const int32_t len = cp[d + 1] - s;
    const int64_t p = base + s + ticket[k];
    const float w = (n > 0.0) ? (float)((double)values[k] / n) : 0.0f;
    if (len == 1) {
      post[p] = make_uint2(local, __float_as_uint(w));
    } else {
      trow[p] = local;
      tval[p] = w;
    }
  }
}

// Workgroup j of slice c handles list entries j, j+G, j+2G, ... in batches of
// NT. Dynamic LDS: two arrays of ceil(S/32) uint32 (bitmap, prefix).
template <int NT>
__global__ __launch_bounds__(NT) void csc_fixup_kernel(
    int64_t dim, int32_t S, int32_t G, const int32_t *__restrict__ flags,
    const int32_t *__restrict__ col_ptr, const int32_t *__restrict__ slice_base,
    const int32_t *__restrict__ mlist, const int32_t *__restrict__ mcount,
    const uint16_t *__restrict__ trow, const float *__restrict__ tval,
    uint2 *__restrict__ post) {
  extern __shared__ uint32_t fx_smem[];
  const int nwords = (S + 31) >> 5;
  uint32_t *bm = fx_smem;
  uint32_t *pre = fx_smem + nwords;
  __shared__ int32_t s_s[NT], s_L[NT];
  __shared__ uint32_t ws[NT / 64];
  if (flags[0] != 0) return;
  const int64_t c = blockIdx.x / G;
  const int64_t g = blockIdx.x % G;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int32_t *cp = col_ptr + c * cp_pitch(dim);
  const int64_t base = slice_base[c];
  const int32_t *ml = mlist + (slice_base[c] / 2 + c);
  const int64_t m = mcount[c];
  const int wpt = (nwords + NT - 1) / NT;  // bitmap words per thread

  for (int64_t kb = 0; g + (int64_t)G * kb < m; kb += NT) {
    const int64_t k = g + (int64_t)G * (kb + t);
    int32_t s = 0, L = 0;
    if (k < m) {
      const int32_t d = ml[k];
      s = cp[d];
      L = cp[d + 1] - s;
    }
    s_s[t] = s;
    s_L[t] = L;
    __syncthreads();

    // lists of 2..64 entries: one wave each, rank by direct comparison
    for (int j = wv; j < NT; j += NT / 64) {
      const int32_t Lj = s_L[j];
      if (Lj < 2 || Lj > 64) continue;
      const int64_t p0 = base + s_s[j];
      uint32_t r = 0xFFFFFFFFu;
      float v = 0.0f;
      if (lane < Lj) {
        r = trow[p0 + lane];
        v = tval[p0 + lane];
      }
      int rank = 0;
      for (int i = 0; i < Lj; ++i) {
        const uint32_t ri = (uint32_t)__builtin_amdgcn_readlane((int)r, i);
        rank += (ri < r) ? 1 : 0;
      }
      if (lane < Lj) post[p0 + rank] = make_uint2(r, __float_as_uint(v));
    }

    // lists of more than 64 entries: the whole workgroup, one list at a time
    for (int j = 0; j < NT; ++j) {
      const int32_t Lj = s_L[j];
      if (Lj <= 64) continue;
      const int64_t p0 = base + s_s[j];
      for (int w = t; w < nwords; w += NT) bm[w] = 0u;
      __syncthreads();
      for (int i = t; i < Lj; i += NT) {
        const uint32_t r = trow[p0 + i];
        atomicOr(&bm[r >> 5], 1u << (r & 31));
      }
      __syncthreads();
      uint32_t cnt = 0;
      for (int q = 0; q < wpt; ++q) {
        const int w = t * wpt + q;
        if (w < nwords) cnt += __popc(bm[w]);
      }
      uint32_t tot;
      uint32_t ex = block_incl_scan<NT>(cnt, ws, &tot) - cnt;
      for (int q = 0; q < wpt; ++q) {
        const int w = t * wpt + q;
        if (w < nwords) {
          pre[w] = ex;
          ex += __popc(bm[w]);
        }
      }
      __syncthreads();
      for (int i = t; i < Lj; i += NT) {
        const uint32_t r = trow[p0 + i];
        const float v = tval[p0 + i];
        const uint32_t w = r >> 5;
        const uint32_t rank = pre[w] + __popc(bm[w] & ((1u << (r & 31)) - 1u));
        post[p0 + rank] = make_uint2(r, __float_as_uint(v));
      }
      __syncthreads();
    }
    __syncthreads();
  }
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

__global__ __launch_bounds__(1024) void heavy_rank_kernel(int32_t cap,
                                                         const int32_t *__restrict__ flags,
                                                         const int32_t *__restrict__ hsel,
                                                         int32_t *__restrict__ heavy) {
  constexpr int NT = 1024;
  __shared__ int32_t s_cd[kCandCap], s_cv[kCandCap];
  __shared__ uint8_t s_sel[kCandCap];
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
  __syncthreads();
  for (int i = t; i < n; i += NT) {
    int rank = 0;
    const int32_t vi = s_cv[i], di = s_cd[i];
    for (int j = 0; j < n; ++j) {
      const int32_t vj = s_cv[j], dj = s_cd[j];
      rank += (vj > vi || (vj == vi && dj < di)) ? 1 : 0;
    }
    s_sel[i] = rank < cap ? 1 : 0;
  }
  __syncthreads();
  for (int i = t; i < n; i += NT) {
    if (!s_sel[i]) continue;
    int pos = 0;
    for (int j = 0; j < n; ++j) pos += (s_sel[j] && s_cd[j] < s_cd[i]) ? 1 : 0;
    heavy[pos] = s_cd[i];
  }
  if (t == 0) heavy[kHeavyMax] = n < cap ? n : cap;
}

// slab of slice s: item j's split-fp16 heavy values in its tile (pre-zeroed)
__global__ __launch_bounds__(256) void slab_scatter_kernel(
    int64_t dim, int32_t pitch, const int32_t *__restrict__ flags,
    const int32_t *__restrict__ heavy, const int32_t *__restrict__ col_ptr,
    const int32_t *__restrict__ slice_base, const uint2 *__restrict__ post,
    uint16_t *__restrict__ slab) {
  const int64_t c = blockIdx.x / kHeavyMax;
  const int h = blockIdx.x % kHeavyMax;
  if (flags[0] != 0 || h >= heavy[kHeavyMax]) return;
  const int32_t d = heavy[h];
  const int32_t *cp = col_ptr + c * cp_pitch(dim);
  const int64_t base = slice_base[c];
  const int32_t b = cp[d], e = cp[d + 1];
  uint16_t *sl = slab + c * (int64_t)pitch * kHeavyRec;
  for (int32_t k = b + threadIdx.x; k < e; k += 256) {
    const uint2 pe = post[base + k];
    if (pe.x < (uint32_t)pitch) {
      uint16_t hi, lo;
      split_fp16(__uint_as_float(pe.y), hi, lo);
      uint16_t *tile = sl + (int64_t)(pe.x >> 4) * kTileHalves;
      tile[heavy_tile_index(pe.x, h, 0)] = hi;
      tile[heavy_tile_index(pe.x, h, 1)] = lo;
    }
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
  e = launch_fill_i32(d.col_ptr, ns * cp_pitch(d.dim), 0, s);
  if (e != hipSuccess) return e;
  e = launch_fill_i32(d.heavy, kHeavyMax + 1, 0, s);
  if (e != hipSuccess) return e;
  e = launch_fill_i32(reinterpret_cast<int32_t *>(d.post + d.nnz), 2 * kPostPad, 0, s);
  if (e != hipSuccess) return e;
  if (g.n_items == 0) return hipSuccess;
  if (d.dense) {
    e = launch_fill_i32(d.gdf, d.dim, 0, s);
    if (e != hipSuccess) return e;
  }
  const unsigned item_blocks = (unsigned)((g.n_items * kLanesPerItem + 255) / 256);
  hipLaunchKernelGGL(csc_count_kernel, dim3(item_blocks), dim3(256), 0, s, g, d.dim, d.indptr,
                     d.indices, d.flags, d.col_ptr, d.ticket);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int32_t hmin = g.S / (2 * kHeavyFracInv) > 2 ? g.S / (2 * kHeavyFracInv) : 2;
  hipLaunchKernelGGL(csc_scan_kernel<1024>, dim3((unsigned)ns), dim3(1024), 0, s, d.dim, d.flags,
                     d.slice_base, d.col_ptr, d.mlist, d.mcount, d.dense ? d.gdf : nullptr, hmin);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(csc_scatter_kernel, dim3(item_blocks), dim3(256), 0, s, g, d.dim, d.indptr,
                     d.indices, d.values, d.norm64, d.flags, d.col_ptr, d.slice_base, d.ticket,
                     d.post, d.trow, d.tval);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  int64_t G = 2048 / ns;
  if (G < 4) G = 4;
  if (G > 256) G = 256;
  const size_t lds = 2 * sizeof(uint32_t) * (size_t)((g.S + 31) / 32);
  hipLaunchKernelGGL(csc_fixup_kernel<256>, dim3((unsigned)(G * ns)), dim3(256), lds, s, d.dim,
                     g.S, (int32_t)G, d.flags, d.col_ptr, d.slice_base, d.mlist, d.mcount, d.trow,
                     d.tval, d.post);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (!d.dense) return hipSuccess;
  const int64_t tg64 = (g.n_items + kHeavyFracInv - 1) / kHeavyFracInv;
  const int32_t tglob = (int32_t)(tg64 > 2 ? tg64 : 2);
  e = launch_fill_i32(d.hsel, 33, 0, s);
  if (e != hipSuccess) return e;
  int64_t hblocks = (d.dim + 255) / 256;
  if (hblocks > 1024) hblocks = 1024;
  hipLaunchKernelGGL(heavy_level_kernel, dim3((unsigned)hblocks), dim3(256), 0, s, d.gdf, d.dim,
                     tglob, d.flags, d.hsel);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(heavy_collect_kernel, dim3((unsigned)hblocks), dim3(256), 0, s, d.gdf, d.dim,
                     tglob, d.flags, d.hsel);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(heavy_rank_kernel, dim3(1), dim3(1024), 0, s, d.heavy_cap, d.flags, d.hsel,
                     d.heavy);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int32_t pitch = slab_pitch(g.S);
  e = launch_fill_i32(reinterpret_cast<int32_t *>(d.slab), ns * (int64_t)pitch * kHeavyRec / 2, 0, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(slab_scatter_kernel, dim3((unsigned)(ns * kHeavyMax)), dim3(256), 0, s,
                     d.dim, pitch, d.flags, d.heavy, d.col_ptr, d.slice_base, d.post, d.slab);
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
    const int32_t *__restrict__ flags, const int32_t *__restrict__ heavy,
    int32_t *__restrict__ lptr, uint3 *__restrict__ lrec, uint16_t *__restrict__ qh) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= n_rows) return;
  const int m = heavy != nullptr ? heavy[kHeavyMax] : 0;
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
    const int hs = m > 0 ? heavy_slot(heavy, m, d) : -1;
    if (FILL) {
      const float v = (n > 0.0) ? (float)((double)values[k] / n) : 0.0f;
      if (hs >= 0) {
        uint16_t hi, lo;
        split_fp16(v, hi, lo);
        uint16_t *tile = qh + (q / kRows) * kTileHalves;
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
    e = launch_fill_i32(reinterpret_cast<int32_t *>(d.qh),
                        (int64_t)d.n_groups * kRows * kHeavyRec / 2, 0, s);
    if (e != hipSuccess) return e;
  }
  const int32_t *heavy = d.dense ? d.heavy : nullptr;
  const unsigned blocks = (unsigned)((d.n_rows + 255) / 256);
  hipLaunchKernelGGL(light_split_kernel<false>, dim3(blocks), dim3(256), 0, s, d.n_rows,
                     d.indptr, d.indices, d.values, d.norm64, d.flags, heavy, d.lptr, d.lrec,
                     d.qh);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(scan_inplace_kernel<1024>, dim3(1), dim3(1024), 0, s, d.lptr,
                     d.n_rows + 1);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(light_split_kernel<true>, dim3(blocks), dim3(256), 0, s, d.n_rows,
                     d.indptr, d.indices, d.values, d.norm64, d.flags, heavy, d.lptr, d.lrec,
                     d.qh);
  return hipGetLastError();
}

}  // namespace sps
