// sps_score.hip -- the score kernel: one item chunk of the exact cosine
// matrix for all query rows.
//
// Page cited: "稀疏嵌入批量相似度计算的工程化实践" (Engineering practice of
// bulk similarity for sparse embeddings): §3.1 (cosine = dot over the shared
// support divided by both norms), §4.4 (items streamed chunk by chunk),
// §2.3 (full float32 output, no top-K).
//
// One workgroup (1024 threads, 16 waves) scores kRows = 16 query rows
// against one slice (<= 2048 items) of the chunk. LDS holds acc[16][Sp]
// (Sp = slice rounded up to 64) as 32-bit fixed point with 30 fraction bits:
// 128 KiB, one workgroup per CU.
//
// Why fixed point: on gfx950 the LDS float atomic (ds_add_f32) sustains about
// 0.3 updates per CU cycle, the 32-bit integer one (ds_add_u32) about 14.
// Why it cannot overflow: both rows are normalised first, so every partial
// sum is bounded by sum_d |q^_d i^_d| <= 1 (Cauchy-Schwarz) and |acc| stays
// below 2^30 plus rounding, inside int32. Integer addition is exact and
// order independent: the result does not depend on how waves interleave.
//
// Dense part (heavy dims): v_mfma_f32_16x16x4f32 with A = 16 rows x 4 dims of
// query values (lane i + 16k holds row i, dim k) and B = 4 dims x 16 items
// of the slice's dense slab (lane j + 16k holds dim k, item j). Item
// 4j + t of each 64-item group feeds the t-th of four MFMAs, so lane l ends
// with rows 4(l/16)..+3 of items 4(l%16)..+3: one float4 per row. fp32
// products and sums in a fixed order over the dims; the sums are added to
// the fixed-point accumulators once at the end.
//
// Sparse part (all other dims): the 16 rows' light entries (dim, value,
// row) are taken in batches of 1024; thread t looks up dim t's posting list
// [col_ptr[d], col_ptr[d+1]) in the slice, a block scan lays the lists end to
// end, and the threads stride through that flat range with U loads in flight
// before their updates: acc[row][j] += rn(fl32(qs * w)) (ds_add_u32), with
// qs = fl32(q_d / |q|) * 2^30, w = fl32(i_d / |i|) and rn rounding to the
// nearest integer (ties up). Posting entries are addressed by 32-bit byte
// offsets from the slice's base (the prepare call keeps nnz below 2^30).
//
// Epilogue: wave w writes row w: out[q, j] = fl32(acc) * 2^-30, 16-byte
// nontemporal stores when aligned (the scores are not re-read, so they
// should not displace posting lists from L2), and the float64 sum of what it
// wrote (a per-chunk checksum; slices are folded in a fixed order).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "sps_device.h"
#include "sps_internal.h"

namespace sps {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// x rounded to the nearest integer, ties upward: floor(x + 0.5) in one
// instruction (|x| <= 2^30 here, so no saturation).
__device__ __forceinline__ int round_fix(float x) {
  int r;
  asm volatile("v_cvt_rpi_i32_f32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

// load at a 32-bit byte offset from a uniform base (base + offset addressing)
template <typename T>
__device__ __forceinline__ T ld_off(const T *base, uint32_t byte_off) {
  return *reinterpret_cast<const T *>(reinterpret_cast<const char *>(base) + byte_off);
}

constexpr int NT = kScoreThreads;
constexpr int NW = NT / 64;
static_assert(NW == kRows, "one wave per query row in the epilogue");
static_assert(kSliceMax <= NW * 2 * 64, "two 64-item groups per wave cover a slice");

template <bool DENSE, int U>
__global__ __launch_bounds__(NT) void score_kernel(const ScoreArgs a, int vec4) {
  extern __shared__ int acc[];
  __shared__ int32_t s_start[NT];    // posting start per batch entry
  __shared__ float s_qv[NT];         // fixed-point-scaled query value per batch entry
  __shared__ int32_t s_row[NT];      // LDS offset of the entry's row
  __shared__ int32_t s_pre[NT + 1];  // flat offsets of the batch's lists
  __shared__ int32_t ws[NW];

  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int64_t grp = blockIdx.x;
  const int ks = blockIdx.y;
  const Geom &g = a.g;
  const int64_t sl = (int64_t)a.chunk * g.n_sub + ks;
  const int64_t ib = g.slice_begin(sl);
  const int32_t slen = (int32_t)(g.slice_end(sl) - ib);
  const int32_t Sp = (g.S + 63) & ~63;
  const int64_t q0 = grp * kRows;
  const int64_t qe = q0 + kRows < a.n_q ? q0 + kRows : a.n_q;

  int4 *acc4 = reinterpret_cast<int4 *>(acc);
  for (int k = t; k < kRows * Sp / 4; k += NT) acc4[k] = make_int4(0, 0, 0, 0);

  // ---- dense part: heavy dims on the matrix cores (registers only) ----
  f32x4 dacc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int u = 0; u < 4; ++u) dacc[i][u] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (DENSE) {
    const int m = a.heavy[kHeavyMax];
    const int m8 = (m + 7) & ~7;  // qh and the slab are zero past m, up to kHeavyMax
    const float *qg = a.qh + grp * (kHeavyMax * kRows);
    const float *sbase = a.slab + sl * (int64_t)kHeavyMax * a.pitch;
    const int kk = lane >> 4, jj = lane & 15;
    for (int h0 = 0; h0 < m8; h0 += 8) {
      float av[2];
      f32x4 sv[2][2];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int h = h0 + 4 * p + kk;
        av[p] = qg[h * kRows + jj];
        const float *srow = sbase + (int64_t)h * a.pitch;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int gp = wv + NW * i;
          sv[p][i] = gp * 64 < Sp ? *reinterpret_cast<const f32x4 *>(srow + gp * 64 + 4 * jj)
                                  : f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
#pragma unroll
      for (int p = 0; p < 2; ++p)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int u = 0; u < 4; ++u)
            dacc[i][u] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[p], sv[p][i][u], dacc[i][u], 0, 0,
                                                              0);
    }
  }
  __syncthreads();  // accumulators zeroed before any update

  // ---- sparse part: the rows' light entries, batch by batch ----
  const int32_t *cps = a.col_ptr + sl * (a.dim + 1);
  const int32_t cb0 = a.slice_base[sl];
  const int32_t snnz = a.slice_base[sl + 1] - cb0 > 0 ? a.slice_base[sl + 1] - cb0 : 0;
  const uint16_t *__restrict__ prow = a.row + cb0;
  const float *__restrict__ pval = a.val + cb0;
  const int32_t e0 = a.lptr[q0], e1 = a.lptr[qe];
  for (int32_t eb = e0; eb < e1; eb += NT) {
    const int n = (e1 - eb) < NT ? (e1 - eb) : NT;
    int32_t s = 0, L = 0;
    if (t < n) {
      const int32_t d = a.ldim[eb + t];
      if ((uint32_t)d < (uint64_t)a.dim) {
        const int32_t lo = cps[d], hi = cps[d + 1];
        s = (int32_t)clamp64(lo, 0, snnz);
        L = (int32_t)clamp64(hi, s, snnz) - s;
      }
      s_qv[t] = a.lval[eb + t];
      s_row[t] = (int32_t)(a.lrow[eb + t] & (kRows - 1)) * Sp;
    }
    s_start[t] = s;
    int32_t total;
    const int32_t incl = block_incl_scan<NT>(L, ws, &total);
    s_pre[t + 1] = incl;
    if (t == 0) s_pre[0] = 0;
    __syncthreads();

    // Wave w walks the flat range [total*w/NW, total*(w+1)/NW), lanes side by
    // side (coalesced loads; a lane crosses few list boundaries). A lane finds
    // its first list by binary search, later ones incrementally.
    const int32_t fb = (int32_t)(((int64_t)total * wv) / NW);
    const int32_t fe = (int32_t)(((int64_t)total * (wv + 1)) / NW);
    int gi = 0;
    {
      int lo = 0, hi = n;  // largest gi with s_pre[gi] <= fb + lane
      const int32_t f = fb + lane;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_pre[mid] <= f) lo = mid;
        else hi = mid;
      }
      gi = lo;
    }
    // the lane's current list, kept in registers
    int32_t t_end = s_pre[gi + 1], t_base = s_start[gi] - s_pre[gi], t_off = s_row[gi];
    float t_qv = s_qv[gi];
    for (int32_t f0 = fb + lane; f0 < fe; f0 += 64 * U) {
      uint32_t pos[U];
      int32_t aoff[U];
      float qv[U];
      bool ok[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int32_t f = f0 + u * 64;
        ok[u] = f < fe;
        if (ok[u] && f >= t_end) {
          do {
            ++gi;
          } while (s_pre[gi + 1] <= f);
          t_end = s_pre[gi + 1];
          t_base = s_start[gi] - s_pre[gi];
          t_off = s_row[gi];
          t_qv = s_qv[gi];
        }
        pos[u] = ok[u] ? (uint32_t)(t_base + f) : 0u;
        aoff[u] = t_off;
        qv[u] = t_qv;
      }
      uint32_t rw[U];
      float w[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        rw[u] = ld_off(prow, pos[u] * 2u);
        w[u] = ld_off(pval, pos[u] * 4u);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (ok[u] && rw[u] < (uint32_t)slen)
          atomicAdd(&acc[aoff[u] + (int)rw[u]], round_fix(qv[u] * w[u]));
      }
    }
    __syncthreads();
  }

  // ---- dense sums into the accumulators ----
  if (DENSE) {
    const int kk = lane >> 4, jj = lane & 15;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int gp = wv + NW * i;
      if (gp * 64 >= Sp) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int *dst = acc + (4 * kk + r) * Sp + gp * 64 + 4 * jj;
#pragma unroll
        for (int u = 0; u < 4; ++u) atomicAdd(dst + u, round_fix(dacc[i][u][r] * kFixScale));
      }
    }
    __syncthreads();
  }

  // ---- epilogue: wave w writes row w ----
  const int64_t q = q0 + wv;
  if (q < a.n_q) {
    const int64_t col0 = ib - g.chunk_begin(a.chunk);
    float *orow = a.out + q * a.ld + col0;
    const bool v4 = vec4 && (col0 % 4 == 0);
    const int4 *arow = reinterpret_cast<const int4 *>(acc + wv * Sp);
    double rs = 0.0;
    for (int j0 = 4 * lane; j0 < slen; j0 += 256) {
      const int4 x = arow[j0 >> 2];
      const f32x4 v = {(float)x.x * kFixInv, (float)x.y * kFixInv, (float)x.z * kFixInv,
                       (float)x.w * kFixInv};
      if (v4 && j0 + 3 < slen) {
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(orow + j0));
        rs += ((double)v[0] + (double)v[1]) + ((double)v[2] + (double)v[3]);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (j0 + u < slen) {
            __builtin_nontemporal_store(v[u], orow + j0 + u);
            rs += (double)v[u];
          }
      }
    }
    double *rsum = g.n_sub == 1 ? a.row_sums : a.rs_part;
    if (rsum != nullptr) {
      rs = wave_sum(rs);
      if (lane == 0) rsum[(g.n_sub == 1 ? 0 : (int64_t)ks * a.n_q) + q] = rs;
    }
  }
}

// row_sums[q] = sum over the chunk's slices, in slice order
__global__ void fold_row_sums_kernel(int64_t n_q, int32_t n_sub, const double *__restrict__ part,
                                     double *__restrict__ row_sums) {
  const int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= n_q) return;
  double s = 0.0;
  for (int k = 0; k < n_sub; ++k) s += part[(int64_t)k * n_q + q];
  row_sums[q] = s;
}

size_t score_lds_bytes(int32_t S) {
  const size_t Sp = (size_t)((S + 63) & ~63);
  return (size_t)kRows * Sp * sizeof(int) + NT * 4 * 3 + (NT + 1) * 4 + NW * 4;
}

static int env_unroll() {
  static int v = -1;
  if (v < 0) {
    v = 4;
    if (const char *e = getenv("SPS_SCORE_UNROLL")) {
      const int x = atoi(e);
      if (x == 2 || x == 4 || x == 8) v = x;
    }
  }
  return v;
}

template <bool DENSE, int U>
static hipError_t launch_t(const ScoreArgs &a, hipStream_t s) {
  const int32_t Sp = (a.g.S + 63) & ~63;
  const size_t dyn = (size_t)kRows * Sp * sizeof(int);
  auto kern = score_kernel<DENSE, U>;
  // dynamic LDS above 64 KiB needs an explicit opt-in per kernel
  static size_t opted = 65536;
  if (dyn > opted) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
    if (e != hipSuccess) return e;
    opted = dyn;
  }
  const int vec4 = (a.ld % 4 == 0) && ((reinterpret_cast<uintptr_t>(a.out) & 15) == 0);
  hipLaunchKernelGGL(kern, dim3((unsigned)a.n_groups, (unsigned)a.g.n_sub), dim3(NT), dyn, s, a,
                     vec4);
  return hipGetLastError();
}

hipError_t launch_score(const ScoreArgs &a, hipStream_t s) {
  if (a.n_groups == 0) return hipSuccess;
  const int u = env_unroll();
  hipError_t e;
  if (a.dense) {
    e = u == 8 ? launch_t<true, 8>(a, s) : (u == 2 ? launch_t<true, 2>(a, s) : launch_t<true, 4>(a, s));
  } else {
    e = u == 8 ? launch_t<false, 8>(a, s)
               : (u == 2 ? launch_t<false, 2>(a, s) : launch_t<false, 4>(a, s));
  }
  if (e != hipSuccess) return e;
  if (a.row_sums != nullptr && a.g.n_sub > 1) {
    hipLaunchKernelGGL(fold_row_sums_kernel, dim3((unsigned)((a.n_q + 255) / 256)), dim3(256), 0,
                       s, a.n_q, a.g.n_sub, a.rs_part, a.row_sums);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace sps
