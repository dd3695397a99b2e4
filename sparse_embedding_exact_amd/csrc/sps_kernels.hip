// sps_kernels.hip -- gfx950 kernels for exact all-pairs sparse cosine.
//
// Page cited throughout: "稀疏嵌入批量相似度计算的工程化实践"
// (Engineering practice of bulk similarity for sparse embeddings).
//
//   row_norm_kernel      §5.2 detail one: L2 norm from the stored nonzeros
//   csr_check_kernel     §3.1 note: canonical CSR (strictly ordered indices)
//   csc_* kernels        per-chunk inverted lists; chunk slicing as in §4.4
//   group_* kernels      query rows merged per workgroup (shared posting reads)
//   score_kernel         §3.1 dot over the shared support, §4.4 normalisation,
//                        §2.3 full float32 output rows
//
// All kernels are wave64. Device-side guards keep every access inside the
// buffers the host sized, whatever the CSR contents.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "sps_internal.h"

namespace sps {

namespace {

__device__ __forceinline__ int64_t clamp64(int64_t v, int64_t lo, int64_t hi) {
  return v < lo ? lo : (v > hi ? hi : v);
}

// inclusive scan over a wave64
template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    T t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Block-wide inclusive scan for NT threads; `ws` is NT/64 elements of LDS.
// Returns the inclusive prefix; *total receives the block sum.
template <int NT, typename T>
__device__ __forceinline__ T block_incl_scan(T v, T *ws, T *total) {
  constexpr int NW = NT / 64;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  T x = wave_incl_scan(v);
  if (lane == 63) ws[w] = x;
  __syncthreads();
  T off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    T s = ws[i];
    if (i < w) off += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return x + off;
}

}  // namespace

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

// ---------------------------------------------------------------------------
// CSR check. flags layout in sps_internal.h.
// ---------------------------------------------------------------------------

// bit: flag bit (1 indptr, 4 index range -> structural; 2 order, 8 non-finite);
// code: reason code kept with the row in the min key (1 indptr, 2 order,
// 3 index range, 4 non-finite).
__device__ __forceinline__ void report(int32_t *flags, int64_t row, int bit, int code) {
  if (bit == 1 || bit == 4) atomicOr(&flags[0], bit);
  else atomicOr(&flags[1], bit);
  const unsigned long long key = ((unsigned long long)row << 3) | (unsigned long long)code;
  atomicMin(reinterpret_cast<unsigned long long *>(flags + 2), key);
}

__global__ __launch_bounds__(256) void csr_check_kernel(int64_t n_rows, int64_t n_cols,
                                                        int64_t nnz,
                                                        const int32_t *__restrict__ indptr,
                                                        const int32_t *__restrict__ indices,
                                                        const float *__restrict__ values,
                                                        int full, int32_t *flags) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r == 0) {
    if (indptr[0] != 0) report(flags, 0, 1, 1);
    if ((int64_t)indptr[n_rows] != nnz) report(flags, n_rows > 0 ? n_rows - 1 : 0, 1, 1);
  }
  if (r >= n_rows) return;
  const int64_t b = indptr[r], e = indptr[r + 1];
  if (b < 0 || e < b || e > nnz) {
    report(flags, r, 1, 1);
    return;
  }
  int32_t prev = -1;
  for (int64_t k = b; k < e; ++k) {
    const int32_t d = indices[k];
    if (d < 0 || (int64_t)d >= n_cols) {
      report(flags, r, 4, 3);
      return;
    }
    if (full) {
      if (d <= prev) report(flags, r, 2, 2);
      if (!isfinite(values[k])) report(flags, r, 8, 4);
    }
    prev = d;
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

__global__ __launch_bounds__(256) void row_norm_kernel(int64_t n_rows, int64_t nnz,
                                                       const int32_t *__restrict__ indptr,
                                                       const float *__restrict__ values,
                                                       const int32_t *__restrict__ flags,
                                                       float *__restrict__ inv32,
                                                       double *__restrict__ norm64) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= n_rows) return;
  const bool bad = flags != nullptr && flags[0] != 0;
  double s = 0.0;
  if (!bad) {
    const int64_t b = clamp64(indptr[r], 0, nnz);
    const int64_t e = clamp64(indptr[r + 1], b, nnz);
    for (int64_t k = b; k < e; ++k) {
      const double v = (double)values[k];
      s += v * v;
    }
  }
  const double n = sqrt(s);
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
// Per-chunk inverted lists. Chunk c holds items [c*C, min((c+1)*C, n)); its
// entries are indptr[c*C] .. indptr[min((c+1)*C, n)) (§4.4 slicing), and its
// inverted lists occupy that same entry range of row[] / val[].
//
//  1. count   : tickets t = atomicAdd(&cnt[c][d], 1) (arbitrary order)
//  2. scan    : col_ptr[c] = exclusive prefix of cnt[c]; list of dims whose
//               list holds >= 2 entries (compacted, ascending)
//  3. scatter : entry -> position col_ptr[c][d] + t; single-entry lists are
//               final, longer lists go to a temporary area
//  4. fixup   : each longer list is put in ascending item order. Item ids
//               are distinct inside one list, so the rank of an entry is the
//               number of smaller ids: a wave compares ids directly for
//               lists up to 64 entries, a workgroup counts bits of an item
//               bitmap (prefix popcounts) for longer ones.
// The result is the unique CSC with ascending item ids per dim, independent
// of the order the atomics were served in.
// ---------------------------------------------------------------------------

__global__ void chunk_base_kernel(int64_t n_items, int64_t nnz, int32_t chunk_size,
                                  int32_t num_chunks, const int32_t *__restrict__ indptr,
                                  int32_t *__restrict__ chunk_base) {
  const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (c > num_chunks) return;
  int64_t i = c * (int64_t)chunk_size;
  if (i > n_items) i = n_items;
  int64_t v = clamp64(indptr[i], 0, nnz);
  chunk_base[c] = (int32_t)v;
}

__global__ __launch_bounds__(256) void csc_count_kernel(int64_t n_items, int64_t dim,
                                                        int64_t nnz, int32_t chunk_size,
                                                        const int32_t *__restrict__ indptr,
                                                        const int32_t *__restrict__ indices,
                                                        const int32_t *__restrict__ flags,
                                                        int32_t *__restrict__ col_ptr,
                                                        int32_t *__restrict__ ticket) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_items || flags[0] != 0) return;
  const int64_t b = indptr[i], e = indptr[i + 1];
  int32_t *cp = col_ptr + (i / chunk_size) * (dim + 1);
  for (int64_t k = b; k < e; ++k) ticket[k] = atomicAdd(&cp[indices[k]], 1);
}

// One workgroup per chunk: exclusive scan of dim+1 counts in place, in tiles
// of 4*NT; plus the compacted list of dims with >= 2 entries. The scan carries
// (count, multi-flag) packed in one 64-bit value: chunk nnz < 2^31 keeps the
// count half from carrying into the flag half.
template <int NT>
__global__ __launch_bounds__(NT) void csc_scan_kernel(int64_t dim,
                                                      const int32_t *__restrict__ flags,
                                                      const int32_t *__restrict__ chunk_base,
                                                      int32_t *__restrict__ col_ptr,
                                                      int32_t *__restrict__ mlist,
                                                      int32_t *__restrict__ mcount) {
  constexpr int TILE = 4 * NT;
  __shared__ int32_t tile[TILE];
  __shared__ int64_t ws[NT / 64];
  const int64_t c = blockIdx.x;
  const int t = threadIdx.x;
  if (flags[0] != 0) {
    if (t == 0) mcount[c] = 0;
    return;
  }
  int32_t *cp = col_ptr + c * (dim + 1);
  int32_t *ml = mlist + (chunk_base[c] / 2 + c);
  const int64_t n = dim + 1;
  int64_t carry = 0;
  for (int64_t base = 0; base < n; base += TILE) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t j = base + k * NT + t;
      tile[k * NT + t] = j < n ? cp[j] : 0;
    }
    __syncthreads();
    int32_t v[4];
    int64_t sum = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[k] = tile[4 * t + k];
      sum += (int64_t)v[k] + ((int64_t)(v[k] >= 2) << 32);
    }
    int64_t tot;
    int64_t incl = block_incl_scan<NT>(sum, ws, &tot);
    int64_t ex = carry + incl - sum;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      tile[4 * t + k] = (int32_t)(ex & 0xFFFFFFFFll);
      if (v[k] >= 2) ml[ex >> 32] = (int32_t)(base + 4 * t + k);
      ex += (int64_t)v[k] + ((int64_t)(v[k] >= 2) << 32);
    }
    carry += tot;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t j = base + k * NT + t;
      if (j < n) cp[j] = tile[k * NT + t];
    }
    __syncthreads();
  }
  if (t == 0) mcount[c] = (int32_t)(carry >> 32);
}

__global__ __launch_bounds__(256) void csc_scatter_kernel(
    int64_t n_items, int64_t dim, int32_t chunk_size, const int32_t *__restrict__ indptr,
    const int32_t *__restrict__ indices, const float *__restrict__ values,
    const double *__restrict__ norm64, const int32_t *__restrict__ flags,
    const int32_t *__restrict__ col_ptr, const int32_t *__restrict__ chunk_base,
    const int32_t *__restrict__ ticket, uint16_t *__restrict__ orow, float *__restrict__ oval,
    uint16_t *__restrict__ trow, float *__restrict__ tval) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_items || flags[0] != 0) return;
  const int64_t c = i / chunk_size;
  const int32_t *cp = col_ptr + c * (dim + 1);
  const int64_t base = chunk_base[c];
  const uint16_t local = (uint16_t)(i - c * (int64_t)chunk_size);
  const double n = norm64[i];
  const int64_t b = indptr[i], e = indptr[i + 1];
  for (int64_t k = b; k < e; ++k) {
    const int32_t d = indices[k];
    const int32_t s = cp[d];
    const int32_t len = cp[d + 1] - s;
    const int64_t p = base + s + ticket[k];
    const float w = (n > 0.0) ? (float)((double)values[k] / n) : 0.0f;
    if (len == 1) {
      orow[p] = local;
      oval[p] = w;
    } else {
      trow[p] = local;
      tval[p] = w;
    }
  }
}

// Workgroup g of chunk c handles list entries g, g+G, g+2G, ... in batches of
// NT. Dynamic LDS: two arrays of ceil(chunk_size/32) uint32 (bitmap, prefix).
template <int NT>
__global__ __launch_bounds__(NT) void csc_fixup_kernel(
    int64_t dim, int32_t chunk_size, int32_t G, const int32_t *__restrict__ flags,
    const int32_t *__restrict__ col_ptr, const int32_t *__restrict__ chunk_base,
    const int32_t *__restrict__ mlist, const int32_t *__restrict__ mcount,
    const uint16_t *__restrict__ trow, const float *__restrict__ tval,
    uint16_t *__restrict__ orow, float *__restrict__ oval) {
  extern __shared__ uint32_t fx_smem[];
  const int nwords = (chunk_size + 31) >> 5;
  uint32_t *bm = fx_smem;
  uint32_t *pre = fx_smem + nwords;
  __shared__ int32_t s_s[NT], s_L[NT];
  __shared__ uint32_t ws[NT / 64];
  if (flags[0] != 0) return;
  const int64_t c = blockIdx.x / G;
  const int64_t g = blockIdx.x % G;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int32_t *cp = col_ptr + c * (dim + 1);
  const int64_t base = chunk_base[c];
  const int32_t *ml = mlist + (chunk_base[c] / 2 + c);
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
      if (lane < Lj) {
        orow[p0 + rank] = (uint16_t)r;
        oval[p0 + rank] = v;
      }
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
        orow[p0 + rank] = (uint16_t)r;
        oval[p0 + rank] = v;
      }
      __syncthreads();
    }
    __syncthreads();
  }
}

hipError_t launch_prepare_items(const ItemsDev &d, hipStream_t s) {
  hipError_t e;
  e = launch_csr_check(d.n_items, d.dim, d.nnz, d.indptr, d.indices, d.values, 0, d.flags, s);
  if (e != hipSuccess) return e;
  e = launch_row_norms(d.n_items, d.nnz, d.indptr, d.values, d.flags, d.inv_norm, d.norm64, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(chunk_base_kernel, dim3((unsigned)((d.num_chunks + 1 + 255) / 256)),
                     dim3(256), 0, s, d.n_items, d.nnz, d.chunk_size, d.num_chunks, d.indptr,
                     d.chunk_base);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  e = launch_fill_i32(d.col_ptr, (int64_t)d.num_chunks * (d.dim + 1), 0, s);
  if (e != hipSuccess) return e;
  if (d.n_items == 0) return hipSuccess;
  const unsigned item_blocks = (unsigned)((d.n_items + 255) / 256);
  hipLaunchKernelGGL(csc_count_kernel, dim3(item_blocks), dim3(256), 0, s, d.n_items, d.dim,
                     d.nnz, d.chunk_size, d.indptr, d.indices, d.flags, d.col_ptr, d.ticket);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(csc_scan_kernel<1024>, dim3((unsigned)d.num_chunks), dim3(1024), 0, s,
                     d.dim, d.flags, d.chunk_base, d.col_ptr, d.mlist, d.mcount);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(csc_scatter_kernel, dim3(item_blocks), dim3(256), 0, s, d.n_items, d.dim,
                     d.chunk_size, d.indptr, d.indices, d.values, d.norm64, d.flags, d.col_ptr,
                     d.chunk_base, d.ticket, d.row, d.val, d.trow, d.tval);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  int G = 2048 / d.num_chunks;
  if (G < 4) G = 4;
  if (G > 256) G = 256;
  const size_t lds = 2 * sizeof(uint32_t) * (size_t)((d.chunk_size + 31) / 32);
  hipLaunchKernelGGL(csc_fixup_kernel<256>, dim3((unsigned)(G * d.num_chunks)), dim3(256), lds,
                     s, d.dim, d.chunk_size, G, d.flags, d.col_ptr, d.chunk_base, d.mlist,
                     d.mcount, d.trow, d.tval, d.row, d.val);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Query row groups: rows [g*R, g*R+R) merged into one ascending dim list with
// R values per dim (0 where a row lacks the dim). Computed once per batch.
// The stored value is the row-normalised query value rounded once to fp32,
// fl32(q_d / |q|) (|q| in float64, §5.2), times 2^30 (exact: a power of two),
// the scale of the fixed-point accumulators of the score kernel.
// ---------------------------------------------------------------------------

constexpr float kFixScale = 1073741824.0f;        // 2^30
constexpr float kFixInv = 9.313225746154785e-10f;  // 2^-30

template <bool FILL>
__global__ __launch_bounds__(256) void group_merge_kernel(
    int64_t n_rows, int64_t nnz, int32_t R, int32_t n_groups, const int32_t *__restrict__ indptr,
    const int32_t *__restrict__ indices, const float *__restrict__ values,
    const double *__restrict__ norm64, const int32_t *__restrict__ flags,
    int32_t *__restrict__ grp_ptr, int32_t *__restrict__ grp_dim, float *__restrict__ grp_val) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= n_groups) return;
  int64_t p[8], e[8];
  double nrm[8];
  const bool bad = flags[0] != 0;
  for (int r = 0; r < 8; ++r) {
    const int64_t q = g * R + r;
    if (r < R && q < n_rows && !bad) {
      p[r] = indptr[q];
      e[r] = indptr[q + 1];
      nrm[r] = norm64[q];
    } else {
      p[r] = 0;
      e[r] = 0;
      nrm[r] = 0.0;
    }
  }
  int64_t out = FILL ? grp_ptr[g] : 0;
  int32_t count = 0;
  for (;;) {
    int32_t dmin = 0x7FFFFFFF;
    for (int r = 0; r < R; ++r)
      if (p[r] < e[r] && indices[p[r]] < dmin) dmin = indices[p[r]];
    if (dmin == 0x7FFFFFFF) break;
    if (FILL) grp_dim[out] = dmin;
    for (int r = 0; r < R; ++r) {
      float v = 0.0f;
      if (p[r] < e[r] && indices[p[r]] == dmin) {
        if (nrm[r] > 0.0) v = (float)((double)values[p[r]] / nrm[r]) * kFixScale;
        ++p[r];
      }
      if (FILL) grp_val[out * R + r] = v;
    }
    ++out;
    ++count;
  }
  if (!FILL) grp_ptr[g + 1] = count;
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

hipError_t launch_prepare_queries(const QueriesDev &d, hipStream_t s) {
  hipError_t e;
  e = launch_csr_check(d.n_rows, d.dim, d.nnz, d.indptr, d.indices, d.values, 0, d.flags, s);
  if (e != hipSuccess) return e;
  e = launch_row_norms(d.n_rows, d.nnz, d.indptr, d.values, d.flags, d.inv_norm, d.norm64, s);
  if (e != hipSuccess) return e;
  e = launch_fill_i32(d.grp_ptr, (int64_t)d.n_groups + 1, 0, s);
  if (e != hipSuccess) return e;
  if (d.n_groups == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((d.n_groups + 255) / 256);
  hipLaunchKernelGGL(group_merge_kernel<false>, dim3(blocks), dim3(256), 0, s, d.n_rows, d.nnz,
                     d.R, d.n_groups, d.indptr, d.indices, d.values, d.norm64, d.flags,
                     d.grp_ptr, d.grp_dim, d.grp_val);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(scan_inplace_kernel<1024>, dim3(1), dim3(1024), 0, s, d.grp_ptr,
                     (int64_t)d.n_groups + 1);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(group_merge_kernel<true>, dim3(blocks), dim3(256), 0, s, d.n_rows, d.nnz,
                     d.R, d.n_groups, d.indptr, d.indices, d.values, d.norm64, d.flags,
                     d.grp_ptr, d.grp_dim, d.grp_val);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Score kernel: one workgroup per group of R query rows, one chunk.
//
// LDS holds acc[R][lenp] as 32-bit fixed point with 30 fraction bits
// (lenp = chunk_len rounded up to 4). The group's merged dim list is taken in
// batches; thread t looks up dim t's posting list [col_ptr[d], col_ptr[d+1])
// in the chunk. Each loaded posting entry (item j, value w = i_d / |i|) is
// added, for every row r of the group holding the dim, as
//     acc[r][j] += rn(fl32(qs_r,d * w)),   qs_r,d = fl32(q_d / |q|) * 2^30,
// with an LDS integer atomic (ds_add_u32). Why integers: on gfx950 the LDS
// float atomic (ds_add_f32) sustains about 0.3 updates per CU cycle while
// ds_add_u32 sustains about 14. Why it cannot overflow: the partial sums of
// normalised rows are bounded by sum |q^_d i^_d| <= 1 (Cauchy-Schwarz), so
// |acc| <= 2^30 plus rounding, inside int32. Integer addition is exact and
// order independent, so the result does not depend on how waves interleave
// (bitwise reproducible). Error per term: fp32 product rounding (<= 2^-24 of
// the term) plus fixed-point rounding (<= 2^-31 absolute).
//
//  - long lists (>= kLongList entries) are walked by the whole workgroup one
//    list at a time: the query values are uniform (scalar registers), and U
//    independent loads per thread are in flight before their atomics;
//  - short lists are laid end to end (block scan of their lengths) and the
//    threads stride through that flat range.
//
// Epilogue: out[q, j] = fl32(acc[r][j]) * 2^-30 over full rows, 16-byte
// nontemporal stores when the row start is aligned (the scores are streamed
// out and not re-read, so they should not displace posting lists from L2);
// optional float64 row sum of the values written.
// ---------------------------------------------------------------------------

constexpr int kLongList = 128;
constexpr int kBatch = 256;

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int R, int NT, int U>
__global__ __launch_bounds__(NT) void score_kernel(
    const int32_t *__restrict__ grp_ptr, const int32_t *__restrict__ grp_dim,
    const float *__restrict__ grp_val, int64_t n_q, int64_t dim,
    const int32_t *__restrict__ col_ptr, const uint16_t *__restrict__ prow_all,
    const float *__restrict__ pval_all, const int32_t *__restrict__ chunk_base, int32_t chunk,
    int32_t chunk_len, int32_t lenp, float *__restrict__ out, int64_t ld,
    double *__restrict__ row_sums, int vec4) {
  constexpr int B = kBatch < NT ? kBatch : NT;  // merged-list entries per batch
  extern __shared__ int acc[];
  __shared__ int32_t s_start[B];   // posting start per batch entry
  __shared__ int32_t s_len[B];     // posting length per batch entry
  __shared__ float s_qv[B * R];    // query values per batch entry
  __shared__ int32_t s_long[B];    // batch entries with long lists (compacted)
  __shared__ int32_t s_sidx[B];    // batch entries with short lists (compacted)
  __shared__ int32_t s_spre[B + 1];  // flat offsets of the short lists
  __shared__ int64_t ws[NT / 64];
  __shared__ double ds[NT / 64];

  const int t = threadIdx.x;
  const int64_t g = blockIdx.x;
  const int64_t q0 = g * R;
  const int32_t cb0 = chunk_base[chunk];
  const int32_t cb1 = chunk_base[chunk + 1];
  const int32_t chunk_nnz = cb1 - cb0 > 0 ? cb1 - cb0 : 0;
  const uint16_t *__restrict__ prow = prow_all + cb0;
  const float *__restrict__ pval = pval_all + cb0;

  int4 *acc4 = reinterpret_cast<int4 *>(acc);
  for (int k = t; k < R * lenp / 4; k += NT) acc4[k] = make_int4(0, 0, 0, 0);

  const int32_t e0 = grp_ptr[g], e1 = grp_ptr[g + 1];
  for (int32_t eb = e0; eb < e1; eb += B) {
    const int n = (e1 - eb) < B ? (e1 - eb) : B;
    int32_t s = 0, L = 0;
    if (t < n) {
      const int32_t d = grp_dim[eb + t];
      if ((uint32_t)d < (uint64_t)dim) {
        const int32_t a = col_ptr[d], b = col_ptr[d + 1];
        s = (int32_t)clamp64(a, 0, chunk_nnz);
        L = (int32_t)clamp64(b, s, chunk_nnz) - s;
      }
#pragma unroll
      for (int r = 0; r < R; ++r) s_qv[t * R + r] = grp_val[(int64_t)(eb + t) * R + r];
    }
    if (t < B) {
      s_start[t] = s;
      s_len[t] = L;
    }
    // compaction: (short-list lengths | short count << 32 | long count << 48)
    const bool is_long = L >= kLongList;
    const bool is_short = L > 0 && !is_long;
    const int64_t key = (is_short ? (int64_t)L : 0) + ((int64_t)is_short << 32) +
                        ((int64_t)is_long << 48);
    int64_t tot;
    const int64_t ex = block_incl_scan<NT>(key, ws, &tot) - key;
    if (is_long) s_long[(ex >> 48) & 0xFFFF] = t;
    if (is_short) {
      const int si = (int)((ex >> 32) & 0xFFFF);
      s_sidx[si] = t;
      s_spre[si + 1] = (int32_t)(ex & 0xFFFFFFFFll) + L;
    }
    if (t == 0) s_spre[0] = 0;
    const int n_long = (int)((tot >> 48) & 0xFFFF);
    const int n_short = (int)((tot >> 32) & 0xFFFF);
    const int32_t short_total = (int32_t)(tot & 0xFFFFFFFFll);
    __syncthreads();

    // ---- long lists: whole workgroup, one list at a time ----
    int32_t rot = 0;  // rotates the thread <-> entry assignment between lists
    for (int h = 0; h < n_long; ++h) {
      const int k = __builtin_amdgcn_readfirstlane(s_long[h]);
      const int32_t st = __builtin_amdgcn_readfirstlane(s_start[k]);
      const int32_t len = __builtin_amdgcn_readfirstlane(s_len[k]);
      float qv[R];
#pragma unroll
      for (int r = 0; r < R; ++r)
        qv[r] = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(s_qv[k * R + r])));
      const int32_t first = (t - rot) & (NT - 1);
      rot = (rot + len) & (NT - 1);
      const uint32_t last = (uint32_t)(st + len - 1);
      for (int32_t f0 = first; f0 < len; f0 += NT * U) {
        uint32_t rw[U];
        float w[U];
        // indices past the list end are clamped to its last entry, so every
        // load is in bounds and unconditional; those lanes skip the adds
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const uint32_t idx = min((uint32_t)(st + f0 + u * NT), last);
          rw[u] = prow[idx];
          w[u] = pval[idx];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (f0 + u * NT >= len || rw[u] >= (uint32_t)chunk_len) continue;
#pragma unroll
          for (int r = 0; r < R; ++r)
            if (qv[r] != 0.0f) atomicAdd(&acc[r * lenp + (int)rw[u]], __float2int_rn(qv[r] * w[u]));
        }
      }
    }

    // ---- short lists: flat range over all of them ----
    int gi = 0;
    for (int32_t f0 = t; f0 < short_total; f0 += NT * U) {
      int32_t p[U];
      int gs[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int32_t f = f0 + u * NT;
        p[u] = -1;
        gs[u] = 0;
        if (f < short_total) {
          while (s_spre[gi + 1] <= f) ++gi;
          const int k = s_sidx[gi];
          p[u] = s_start[k] + (f - s_spre[gi]);
          gs[u] = k;
        }
      }
      uint32_t rw[U];
      float w[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (p[u] >= 0) {
          rw[u] = prow[p[u]];
          w[u] = pval[p[u]];
        } else {
          rw[u] = 0xFFFFFFFFu;
          w[u] = 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (rw[u] >= (uint32_t)chunk_len) continue;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float qv = s_qv[gs[u] * R + r];
          if (qv != 0.0f) atomicAdd(&acc[r * lenp + (int)rw[u]], __float2int_rn(qv * w[u]));
        }
      }
    }
    (void)n_short;
    __syncthreads();
  }
  __syncthreads();

  const int lane = t & 63, wv = t >> 6;
  for (int r = 0; r < R; ++r) {
    const int64_t q = q0 + r;
    if (q >= n_q) break;
    float *orow = out + q * ld;
    const int *arow = acc + r * lenp;
    double rs = 0.0;
    int jstart = 0;
    if (vec4) {
      const int n4 = chunk_len >> 2;
      const int4 *a4 = reinterpret_cast<const int4 *>(arow);
      f32x4 *o4 = reinterpret_cast<f32x4 *>(orow);
      for (int k = t; k < n4; k += NT) {
        const int4 a = a4[k];
        const f32x4 v = {(float)a.x * kFixInv, (float)a.y * kFixInv, (float)a.z * kFixInv,
                         (float)a.w * kFixInv};
        __builtin_nontemporal_store(v, o4 + k);
        rs += ((double)v.x + (double)v.y) + ((double)v.z + (double)v.w);
      }
      jstart = n4 << 2;
    }
    for (int j = jstart + t; j < chunk_len; j += NT) {
      const float v = (float)arow[j] * kFixInv;
      __builtin_nontemporal_store(v, &orow[j]);
      rs += (double)v;
    }
    if (row_sums) {
      rs = wave_sum(rs);
      if (lane == 0) ds[wv] = rs;
      __syncthreads();
      if (t == 0) {
        double tot = 0.0;
        for (int i = 0; i < NT / 64; ++i) tot += ds[i];
        row_sums[q] = tot;
      }
      __syncthreads();
    }
  }
}

static int score_nt() {
  static int v = -1;
  if (v < 0) {
    v = 256;
    if (const char *e = getenv("SPS_SCORE_THREADS")) {
      const int x = atoi(e);
      if (x == 256 || x == 512 || x == 1024) v = x;
    }
  }
  return v;
}

static int score_unroll() {
  static int v = -1;
  if (v < 0) {
    v = 8;
    if (const char *e = getenv("SPS_SCORE_UNROLL")) {
      const int x = atoi(e);
      if (x == 4 || x == 8) v = x;
    }
  }
  return v;
}

size_t score_lds_bytes(int R, int32_t chunk_len) {
  const size_t NT = 1024, B = kBatch;  // largest workgroup bounds the static part
  const size_t lenp = (size_t)((chunk_len + 3) & ~3);
  const size_t dyn = (size_t)R * lenp * sizeof(float);
  const size_t stat = B * 4 * 4 + (B + 1) * 4 + B * (size_t)R * 4 + (NT / 64) * 16 + 64;
  return dyn + stat;
}

int score_max_rows(int32_t chunk_len, size_t lds_limit) {
  for (int R = 8; R >= 1; R >>= 1)
    if (score_lds_bytes(R, chunk_len) <= lds_limit) return R;
  return 0;
}

template <int R, int NT, int U>
static hipError_t launch_score_t(const ScoreArgs &a, hipStream_t s) {
  const int32_t lenp = (a.chunk_len + 3) & ~3;
  const size_t dyn = (size_t)R * lenp * sizeof(int);
  auto kern = score_kernel<R, NT, U>;
  // dynamic LDS above 64 KiB needs an explicit opt-in per kernel
  static size_t opted = 65536;
  if (dyn > opted) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
    if (e != hipSuccess) return e;
    opted = dyn;
  }
  const int vec4 = (a.ld % 4 == 0) && ((reinterpret_cast<uintptr_t>(a.out) & 15) == 0);
  hipLaunchKernelGGL(kern, dim3((unsigned)a.n_groups), dim3(NT), dyn, s, a.grp_ptr, a.grp_dim,
                     a.grp_val, a.n_q, a.dim, a.col_ptr, a.row, a.val, a.chunk_base,
                     a.chunk, a.chunk_len, lenp, a.out, a.ld, a.row_sums, vec4);
  return hipGetLastError();
}

template <int R>
static hipError_t launch_score_r(const ScoreArgs &a, hipStream_t s) {
  const int nt = score_nt(), u = score_unroll();
  if (nt == 1024) return u == 8 ? launch_score_t<R, 1024, 8>(a, s) : launch_score_t<R, 1024, 4>(a, s);
  if (nt == 512) return u == 8 ? launch_score_t<R, 512, 8>(a, s) : launch_score_t<R, 512, 4>(a, s);
  return u == 8 ? launch_score_t<R, 256, 8>(a, s) : launch_score_t<R, 256, 4>(a, s);
}

hipError_t launch_score(const ScoreArgs &a, hipStream_t s) {
  if (a.n_groups == 0) return hipSuccess;
  switch (a.R) {
    case 1: return launch_score_r<1>(a, s);
    case 2: return launch_score_r<2>(a, s);
    case 4: return launch_score_r<4>(a, s);
    case 8: return launch_score_r<8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sps
