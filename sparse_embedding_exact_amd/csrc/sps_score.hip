// sps_score.hip -- the score kernel: one item chunk of the exact cosine
// matrix for all query rows.
//
// Page cited: "稀疏嵌入批量相似度计算的工程化实践" (Engineering practice of
// bulk similarity for sparse embeddings): §3.1 (cosine = dot over the shared
// support divided by both norms), §4.4 (items streamed chunk by chunk),
// §2.3 (full float32 output, no top-K).
//
// One workgroup (512 threads, 8 waves) scores kRows = 8 query rows against
// one slice (<= 2048 items) of the chunk. LDS holds acc[8][Sp] (Sp = slice
// rounded up to 128) as 32-bit fixed point with 30 fraction bits: 64 KiB, so
// two workgroups share a CU and one's stores overlap the other's gathers.
//
// Why fixed point: on gfx950 the LDS float atomic (ds_add_f32) sustains about
// 0.3 updates per CU cycle, the 32-bit integer one (ds_add_u32) about 14.
// Why it cannot overflow: both rows are normalised first, so every partial
// sum is bounded by sum_d |q^_d i^_d| <= 1 (Cauchy-Schwarz) and |acc| stays
// below 2^30 plus rounding, inside int32. Integer addition is exact and
// order independent: the result does not depend on how waves interleave.
//
// Dense part (heavy dims): v_mfma_f32_4x4x1f32, 16 independent 4x4x1 blocks
// per instruction (lanes 4b..4b+3 form block b; lane l's result i is
// A[lane 4(l/4) + i] * B[lane l]). Every lane supplies one item of the
// slice's dense slab as B and lane m the value of query row m % 4 (or
// 4 + m % 4) as A, so one B load feeds two MFMAs (rows 0-3, rows 4-7) and
// lane l accumulates all 8 rows of its items. fp32 products and sums in a
// fixed order over the dims; the sums, rounded once to fixed point, start
// the accumulators.
//
// Sparse part (all other dims): the 8 rows' light entries (dim, value,
// row) are taken in batches of 512; thread t looks up entry t's posting list
// [col_ptr[d], col_ptr[d+1]) in the slice. Lists are cut into segments of
// 16 postings, a block scan numbers the segments and a table in LDS names
// each one's list, so 16 lanes take one segment with no search: lane i of a
// segment handles posting 16k + i of its list, loads (item, w) and applies
// acc[row][item] += rn(fl32(qs * w)) (ds_add_u32), with qs = fl32(q_d / |q|)
// * 2^30, w = fl32(i_d / |i|) and rn rounding to the nearest integer (ties
// up). Posting entries are addressed by 32-bit byte offsets from the slice's
// base (the prepare call keeps nnz below 2^30).
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
static_assert(kRows == 8, "the dense part maps two 4-row MFMA blocks");
static_assert(kSliceMax <= NW * 256, "256 items per wave cover a slice");
static_assert(kRows * kHeavyMax / 4 <= NT, "one float4 of heavy query values per thread");
// Sparse part: posting lists are cut into segments of kSeg entries, one per
// 16 lanes; a segment is named by (list, index) in 16 bits.
constexpr int kSeg = 16;
constexpr int kSegMax = 2048;  // segments per round (LDS table)
static_assert(NT * ((kSliceMax + kSeg - 1) / kSeg) <= 65536, "segment names fit 16 bits");
static_assert((kSliceMax + kSeg - 1) / kSeg <= 128, "segment index fits 7 bits");

template <bool DENSE, int U>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) void score_kernel(
    const ScoreArgs a, int vec4) {
  extern __shared__ int acc[];
  __shared__ int4 s_rec[NT];          // per batch entry: posting start, length, row offset, value
  __shared__ uint16_t s_seg[kSegMax];  // segment table of a round
  __shared__ int32_t ws[NW];
  __shared__ __align__(16) float s_qh[DENSE ? kRows * kHeavyMax : 4];  // the rows' heavy values

  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int64_t grp = blockIdx.x;
  const int ks = blockIdx.y;
  const Geom &g = a.g;
  const int64_t sl = (int64_t)a.chunk * g.n_sub + ks;
  const int64_t ib = g.slice_begin(sl);
  const int32_t slen = (int32_t)(g.slice_end(sl) - ib);
  const int32_t Sp = slab_pitch(g.S);
  const int64_t q0 = grp * kRows;
  const int64_t qe = q0 + kRows < a.n_q ? q0 + kRows : a.n_q;

  // First batch of light entries (see the sparse part): descriptors are
  // fetched before the dense part so that their two dependent loads (entry,
  // then posting range) overlap it.
  const int32_t *cps = a.col_ptr + sl * (a.dim + 1);
  const int32_t cb0 = a.slice_base[sl];
  const int32_t snnz = a.slice_base[sl + 1] - cb0 > 0 ? a.slice_base[sl + 1] - cb0 : 0;
  const int32_t e0 = a.lptr[q0], e1 = a.lptr[qe];
  int32_t b_s = 0, b_L = 0, b_row = 0;
  float b_qv = 0.f;
  auto fetch = [&](int32_t eb) {
    b_s = 0;
    b_L = 0;
    if (eb + t < e1) {
      const int32_t d = a.ldim[eb + t];
      b_qv = a.lval[eb + t];
      b_row = (int32_t)(a.lrow[eb + t] & (kRows - 1)) * Sp;
      if ((uint32_t)d < (uint64_t)a.dim) {
        const int32_t lo = cps[d], hi = cps[d + 1];
        b_s = (int32_t)clamp64(lo, 0, snnz);
        b_L = (int32_t)clamp64(hi, b_s, snnz) - b_s;
        b_L = b_L < kSliceMax ? b_L : kSliceMax;  // a slice holds a dim at most once per item
      }
    }
  };
  fetch(e0);

  // ---- dense part: heavy dims on the matrix cores ----
  // Wave w owns items [256 w, 256 w + 256) of the slice, 4 per lane. Dims are
  // taken 4 at a time, the next 4 loaded while the current ones are
  // multiplied. qh and the slab hold zeros from the last heavy dim up to
  // kHeavyMax, so rounding the dim count up to 8 only adds exact zeros. The
  // sums, rounded to fixed point, are the accumulators' initial values.
  const int32_t wcol = wv * 256;
  if (DENSE) {
    const int mr = (a.heavy[kHeavyMax] + 7) & ~7;
    const float *sb = a.slab + sl * (int64_t)kHeavyMax * a.pitch + (wcol < Sp ? wcol : 0) + 4 * lane;
    f32x4 sv[2][4];
    auto load = [&](int b, int h0) {
#pragma unroll
      for (int p = 0; p < 4; ++p)
        sv[b][p] = *reinterpret_cast<const f32x4 *>(sb + (int64_t)(h0 + p) * a.pitch);
    };
    if (mr > 0) load(0, 0);
    if (t < kRows * kHeavyMax / 4)
      reinterpret_cast<f32x4 *>(s_qh)[t] =
          reinterpret_cast<const f32x4 *>(a.qh + grp * (kRows * kHeavyMax))[t];
    __syncthreads();
    f32x4 dacc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int u = 0; u < 4; ++u) dacc[i][u] = f32x4{0.f, 0.f, 0.f, 0.f};
    // A operands: lane m supplies query row m % 4 (block 0) and 4 + m % 4
    // (block 1), four dims per LDS read.
    const float *qa = s_qh + (lane & 3) * kHeavyMax;
    auto mma = [&](int b, int h0) {
      const f32x4 alo = *reinterpret_cast<const f32x4 *>(qa + h0);
      const f32x4 ahi = *reinterpret_cast<const f32x4 *>(qa + 4 * kHeavyMax + h0);
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          dacc[0][u] = __builtin_amdgcn_mfma_f32_4x4x1f32(alo[p], sv[b][p][u], dacc[0][u], 0, 0, 0);
          dacc[1][u] = __builtin_amdgcn_mfma_f32_4x4x1f32(ahi[p], sv[b][p][u], dacc[1][u], 0, 0, 0);
        }
    };
    if (wcol < Sp) {
      for (int h0 = 0; h0 < mr; h0 += 8) {
        load(1, h0 + 4);
        mma(0, h0);
        if (h0 + 8 < mr) load(0, h0 + 8);
        mma(1, h0 + 4);
      }
      // lane l holds rows 4b + i of items 4l + u in dacc[b][u][i]
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        const int b = r >> 2, i = r & 3;
        reinterpret_cast<int4 *>(acc + r * Sp + wcol)[lane] =
            make_int4(round_fix(dacc[b][0][i] * kFixScale), round_fix(dacc[b][1][i] * kFixScale),
                      round_fix(dacc[b][2][i] * kFixScale), round_fix(dacc[b][3][i] * kFixScale));
      }
    }
  } else {
    int4 *acc4 = reinterpret_cast<int4 *>(acc);
    for (int k = t; k < kRows * Sp / 4; k += NT) acc4[k] = make_int4(0, 0, 0, 0);
  }
  __syncthreads();  // accumulators initialised before any sparse update

  // ---- sparse part: the rows' light entries, batch by batch ----
  const uint16_t *__restrict__ prow = a.row + cb0;
  const float *__restrict__ pval = a.val + cb0;
  for (int32_t eb = e0; eb < e1; eb += NT) {
    // list record of entry t: posting start, length, LDS row offset, value
    s_rec[t] = make_int4(b_s, b_L, b_row, __float_as_int(b_qv));
    const int32_t nseg = (b_L + kSeg - 1) / kSeg;
    int32_t total;
    const int32_t sp0 = block_incl_scan<NT>(nseg, ws, &total) - nseg;  // barrier inside
    if (eb + NT < e1) fetch(eb + NT);  // next batch's descriptors, in flight during this one
    for (int32_t r0 = 0; r0 < total; r0 += kSegMax) {
      // segment table of the round: list id and segment index within the list
      const int32_t sb = sp0 > r0 ? sp0 : r0;
      const int32_t se = sp0 + nseg < r0 + kSegMax ? sp0 + nseg : r0 + kSegMax;
      for (int32_t sg = sb; sg < se; ++sg) s_seg[sg - r0] = (uint16_t)((t << 7) | (sg - sp0));
      __syncthreads();
      const int32_t nr = total - r0 < kSegMax ? total - r0 : kSegMax;
      // wave w takes segment quads w, w + NW, ...; lanes 16i..16i+15 segment i of a quad
      for (int32_t k0 = wv; 4 * k0 < nr; k0 += NW * U) {
        uint32_t pos[U];
        int32_t aoff[U];
        float qv[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int32_t sg = 4 * (k0 + NW * u) + (lane >> 4);
          const bool in = sg < nr;
          const uint32_t desc = s_seg[in ? sg : 0];
          const int4 rec = s_rec[desc >> 7];
          const int32_t j = (int32_t)(desc & 127) * kSeg + (lane & 15);
          ok[u] = in && j < rec.y;
          pos[u] = ok[u] ? (uint32_t)(rec.x + j) : 0u;
          aoff[u] = rec.z;
          qv[u] = __int_as_float(rec.w);
        }
        uint16_t rw[U];
        float w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          rw[u] = ld_off(prow, pos[u] * 2u);
          w[u] = ld_off(pval, pos[u] * 4u);
        }
        // all 2U loads are in flight before the first is waited on (keeps the
        // compiler from sinking a load into the masked update below it)
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) asm volatile("" ::"v"(rw[u]), "v"(w[u]));
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (ok[u] && (int32_t)rw[u] < slen)
            atomicAdd(&acc[aoff[u] + (int)rw[u]], round_fix(qv[u] * w[u]));
        }
      }
      __syncthreads();
    }
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
  const size_t Sp = (size_t)slab_pitch(S);
  return (size_t)kRows * Sp * sizeof(int) + NT * 16 + kSegMax * 2 + NW * 4 +
         kRows * kHeavyMax * 4;
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
  const int32_t Sp = slab_pitch(a.g.S);
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
