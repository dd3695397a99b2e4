// sps_score.hip -- the score kernel: one item chunk of the exact cosine
// matrix for all query rows.
//
// Page cited: "稀疏嵌入批量相似度计算的工程化实践" (Engineering practice of
// bulk similarity for sparse embeddings): §3.1 (cosine = dot over the shared
// support divided by both norms), §4.4 (items streamed chunk by chunk),
// §2.3 (full float32 output, no top-K).
//
// One workgroup (512 threads, 8 waves) scores two groups of kRows = 16 query
// rows, one after the other, against one slice (<= 1024 items) of the chunk.
// LDS holds acc[16][Lp] (Lp = slice rounded up to 128, plus 4 against bank
// conflicts) as 32-bit fixed point with 30 fraction bits: 64 KiB, so two
// workgroups share a CU. Workgroups are numbered slice-fastest (see the
// kernel).
//
// Why fixed point: on gfx950 the LDS float atomic (ds_add_f32) sustains about
// 0.3 updates per CU cycle, the 32-bit integer one (ds_add_u32) about 14.
// Why it cannot overflow: both rows are normalised first, so every partial
// sum is bounded by sum_d |q^_d i^_d| <= 1 (Cauchy-Schwarz) and |acc| stays
// below 2^30 plus rounding, inside int32. Integer addition is exact and
// order independent: the result does not depend on how waves interleave.
//
// Dense part (heavy dims): v_mfma_f32_16x16x32_f16 on values split in two
// fp16 halves (hi, lo) after scaling by 2^15, so the dot of two values is
// hi.hi + (hi.lo + lo.hi) / 2048 up to 3 * 2^-22 of |x y| (the lo.lo term is
// dropped). A is the 16 rows' values on a block of 32 heavy dims, B the
// slab's 16 items of a tile, both stored in the MFMA operand order (A[i][k]
// in lane i + 16 (k / 8), element k % 8). Each slab value loaded feeds all 16
// rows of both row groups. Per block, fp32 sums rounded once to fixed point;
// the blocks' sums start the accumulators (one to four blocks, chosen per
// corpus by the prepare).
//
// Sparse part (all other dims): the 16 rows' light entries (dim, value,
// row) are taken in batches of 1024, two per thread; each looks up its
// posting list [col_ptr[d], col_ptr[d+1]) in the slice. Lists are cut into
// segments of 16 postings, a block scan numbers the segments and an LDS
// table records each one (first posting, value, row, length), so 8 lanes
// take one segment with no search: lane i handles postings 2i and 2i + 1 of
// it, loads both (item, w) pairs with one 16-byte load and applies
// acc[row][item] += rn(fl32(qs * w)) (ds_add_u32) for each, with qs =
// fl32(q_d / |q|) * 2^30, w = fl32(i_d / |i|) and rn rounding to the nearest
// integer (ties up). (The vector-memory data path, not the LDS atomics, is
// what limits this loop, so fewer and wider loads pay.)
//
// Epilogue: wave w writes rows w and w + 8: out[q, j] = fl32(acc) * 2^-30,
// 16-byte nontemporal stores when aligned (the scores are not re-read, so
// they should not displace posting lists from L2), and the float64 sum of
// what it wrote (a per-chunk checksum; slices are folded in a fixed order).
// That sum is exact in any order: every score written is an integer multiple
// of 2^-30 below 2 in magnitude and a chunk row holds at most 2^20 of them,
// so every partial sum is an integer multiple of 2^-30 below 2^21, which a
// float64 holds exactly. The lanes' sums are added with DPP lane moves, not
// through LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "sps_device.h"
#include "sps_internal.h"

namespace sps {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));

// dense sums are of values scaled by kHeavyScale on both sides
constexpr float kDenseToFix = kFixScale / (kHeavyScale * kHeavyScale);  // 1
static_assert(kDenseToFix == 1.0f, "dense sums are already in fixed-point units");

// x rounded to the nearest integer, ties upward: floor(x + 0.5) in one
// instruction (|x| <= 2^30 here, so no saturation).
// (Not volatile: a pure register operation, which the scheduler may move
// like any other; a volatile one orders every memory access around it.)
__device__ __forceinline__ int round_fix(float x) {
  int r;
  asm("v_cvt_rpi_i32_f32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

// two consecutive 8-byte postings (item, value, item, value) with one
// 16-byte load from an 8-byte aligned address (global memory accesses need
// only 4-byte alignment on this target)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_a8 __attribute__((ext_vector_type(4), aligned(8)));
__device__ __forceinline__ u32x4 ld_pair(const uint2 *base, uint32_t byte_off) {
  return *reinterpret_cast<const u32x4_a8 *>(reinterpret_cast<const char *>(base) + byte_off);
}

// four consecutive 4-byte postings with one 16-byte load (4-byte aligned)
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
__device__ __forceinline__ u32x4 ld_quad4(const uint32_t *base, uint32_t byte_off) {
  return *reinterpret_cast<const u32x4_a4 *>(reinterpret_cast<const char *>(base) + byte_off);
}

constexpr int kOutExact = kModeExact, kOutHalf = kModeHalf, kOutThreshold = kModeThreshold;

constexpr int NT = kScoreThreads;
constexpr int NW = NT / 64;
constexpr int kBatch = 2 * NT;  // light entries per batch, two per thread
constexpr int kGroups = 2;      // row groups per workgroup (they share the slab loads)
static_assert(kRows % NW == 0, "whole rows per wave in the epilogue");
static_assert(kSliceMax <= NW * 128, "128 items per wave cover a slice");
static_assert(kRows == 16 && kHeavyBlock == 32, "one 16x16x32 MFMA tile covers the rows and a block");
// Sparse part: posting lists are cut into segments of kSeg entries, one per
// 16 lanes, described in an LDS table.
constexpr int kSeg = 16;
constexpr int kSegMax = 1024;        // segments per round (the LDS left beside two 64 KiB accumulators)
constexpr int kSegPad = 16 * NW * 2;  // at least one walk step past the end (SPI * NW * U segments)
static_assert(kRows * kSliceMax * 4 < (1 << 27), "row byte offset fits the segment record");

// MODE kOutExact: fp32 scores. kOutHalf: the reduced-precision variant (item
// values as fp16, scores written as fp16; see sps_cosine_chunk_half): 4-byte
// postings, four per lane and load, the slab's hi halves only, fp16 output.
// kOutThreshold: the exact scores, of which only those >= a.threshold are
// written, as (row, item, score) hits (see sps_cosine_chunk_threshold).
// The workgroup's LDS, declared once in the kernel (the body below is
// instantiated twice in it): the accumulators, the segment table of a round
// (first posting, query value, and the LDS byte offset of the row << 5 |
// postings in the segment, 1..16, 0 padding the table past its last
// segment), the block scan's two buffers, and the threshold epilogue's hits
// per wave and first hit position.
struct ScoreLds {
  int *acc;
  uint32_t *s_spos, *s_sqv, *s_smeta;
  int32_t (*ws)[NW];
  int32_t *s_wtot;
  unsigned long long *s_hbase;
  int *sink;  // one slot per lane for the walk's masked-off adds
};

template <bool DENSE, int MODE>
__device__ __forceinline__ void score_body(const ScoreArgs &a, int vec4, const ScoreLds &L,
                                           int nblk) {
  constexpr bool HALF = MODE == kOutHalf;
  // segment groups per wave per walk step: three where the dense part runs
  // (its corpora have long lists), two otherwise (the edge corpus: no heavy
  // dims, short lists)
  constexpr int U = HALF || !DENSE ? 2 : 3;
  constexpr int PPL = HALF ? 4 : 2;         // postings per lane (one 16-byte load)
  constexpr int LPS = kSeg / PPL;           // lanes per segment
  constexpr int SPI = 64 / LPS;             // segments per wave per load
  static_assert(SPI * NW * U <= kSegPad, "the segment table pads one walk step per wave");
  int *const acc = L.acc;
  uint32_t *const s_spos = L.s_spos, *const s_sqv = L.s_sqv, *const s_smeta = L.s_smeta;
  int32_t (*const ws)[NW] = L.ws;
  int32_t *const s_wtot = L.s_wtot;
  unsigned long long &s_hbase = *L.s_hbase;

  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const Geom &g = a.g;
  // Slice-fastest order: consecutive workgroups take the slices of one pair
  // of row groups, and workgroups are dealt to the 8 XCDs in turn, so with
  // n_sub dividing 8 each XCD keeps to the same slice of the chunk (its
  // posting lists and slab stay in that XCD's L2) while the rows written at
  // any time span whole output rows.
  const int64_t grp0 = (blockIdx.x / g.n_sub) * kGroups;
  const int ks = (int)(blockIdx.x % g.n_sub);
  const int ng = (int)(a.n_groups - grp0 < kGroups ? a.n_groups - grp0 : kGroups);  // 1 or 2
  const int64_t sl = (int64_t)a.chunk * g.n_sub + ks;
  const int64_t ib = g.slice_begin(sl);
  const int32_t slen = (int32_t)(g.slice_end(sl) - ib);
  const int32_t Sp = slab_pitch(g.S);  // slab row pitch (items)
  const int32_t Lp = acc_pitch(g.S);   // accumulator row pitch (ints)

  const int4 dix = a.dinfo[sl];  // the slice's dim index (uniform)
  const uint4 *__restrict__ dtab = a.dtab + dix.x;
  const int32_t cb0 = a.slice_base[sl];
  const int32_t snnz = a.slice_base[sl + 1] - cb0 > 0 ? a.slice_base[sl + 1] - cb0 : 0;
  // light entries of group gi: [ge[gi], ge[gi + 1]) (the rows are consecutive)
  int32_t ge[kGroups + 1];
#pragma unroll
  for (int gi = 0; gi <= kGroups; ++gi) {
    const int64_t q = (grp0 + (gi < ng ? gi : ng)) * kRows;
    ge[gi] = a.lptr[q < a.n_q ? q : a.n_q];
  }

  // Batch descriptors (see the sparse part): entries eb + t and eb + t + NT
  // of a batch [eb, ee). Three stages, so that other loads can be issued
  // between them and no arithmetic on a loaded value forces an early wait:
  // the entry records (dim, value, row); then the dependent posting ranges;
  // then the range arithmetic. The first batch of each group is fetched at
  // the start, so both groups' lookups overlap the dense part.
  struct Raw {
    uint3 rec[2];  // (dim, value bits, row in group)
    uint4 bkt[2];  // the dim's home bucket in the slice's index
    bool ok[2];
  };
  struct Desc {
    int32_t s[2], L[2], row[2];
    float qv[2];
  };
  auto fetch_entries = [&](Raw &r, int32_t eb, int32_t ee) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int32_t e = eb + t + i * NT;
      r.ok[i] = e < ee;
      // a readable entry (the light arrays hold at least one) when e is past the end
      r.rec[i] = a.lrec[e < ee ? e : (ee > 0 ? ee - 1 : 0)];
    }
  };
  // (the dim is checked here, so that it is not kept until the arithmetic)
  auto fetch_ranges = [&](Raw &r) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      r.ok[i] = r.ok[i] && r.rec[i].x < (uint64_t)a.dim;
      // the home bucket of the dim: one 16-byte load; most lookups end there
      r.bkt[i] = dtab[dim_bucket(r.rec[i].x, (uint32_t)dix.y)];
    }
  };
  auto finish_ranges = [&](const Raw &r, Desc &b) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t d = r.rec[i].x;
      int32_t st = 0, L = 0;
      int res = r.ok[i] ? dim_probe(r.bkt[i], d, dix.z != 0, st, L) : 0;
      if (res < 0) {  // a full home bucket: follow the chain
        const uint32_t nb = (uint32_t)dix.y;
        uint32_t bk = dim_bucket(d, nb);
        for (uint32_t k = 1; k < nb && res < 0; ++k) {
          bk = bk + 1 == nb ? 0u : bk + 1;
          res = dim_probe(dtab[bk], d, dix.z != 0, st, L);
        }
      }
      if (res != 1) st = L = 0;
      // (clamped to the slice's postings in 32-bit arithmetic: 0 <= s <= snnz,
      // so snnz - s cannot overflow)
      const int32_t s0 = min(max(st, 0), snnz);
      L = min(max(L, 0), snnz - s0);
      b.s[i] = s0;
      b.L[i] = L < kSliceMax ? L : kSliceMax;  // a slice holds a dim once per item
      b.row[i] = (int32_t)(r.rec[i].z & (kRows - 1));
      b.qv[i] = __uint_as_float(r.rec[i].y);
    }
  };
  auto batch_end = [&](int32_t eb, int32_t ee) { return ee - eb < kBatch ? ee : eb + kBatch; };
  Raw r0, r1;
  const int32_t f0 = batch_end(ge[0], ge[1]), f1 = batch_end(ge[1], ge[2]);
  fetch_entries(r0, ge[0], f0);
  fetch_entries(r1, ge[1], f1);

  // ---- dense part: heavy dims on the matrix cores ----
  // Wave w owns items [128 w, 128 w + 128) of the slice as 8 tiles of 16.
  // Per tile and row group, three v_mfma_f32_16x16x32_f16 over a block of
  // 32 heavy dims: main = hi.hi and cross = hi.lo + lo.hi of the split
  // values, so that the dot of the scaled values is main + cross / 2048
  // (fp32). Both sides carry 2^15, so that sum is already in the
  // accumulators' fixed-point units (2^30): rounded once, it is their
  // initial value. Group 0's is written to LDS at once, group 1's waits in
  // registers. Each slab tile loaded serves both groups.
  const int32_t wcol = wv * 128;
  constexpr int kTiles = 8, kHalf = 4;  // tiles per wave, loaded in two halves
  h16x8 a_hi[kGroups], a_lo[kGroups], b_hi[kHalf], b_lo[kHalf];
  int32_t dpend[kTiles][4];  // group 1's initial values, fixed point
  const bool wdense = DENSE && wcol < Sp;
  // A: lane l holds row l%16, dims 8(l/16)..+7 (hi, lo); B: item l%16 of the
  // tile, the same dims. Both are tiles in the MFMA operand order. The loads
  // are unconditional (a wave past the slice loads tile 0 and drops it), so
  // that the counter waits below see one path.
  static_assert(kTileHalves == 2 * 64 * 8, "a tile is one 16-byte load per lane per part");
  const h16x8 *st = reinterpret_cast<const h16x8 *>(
      a.slab + (sl * (int64_t)a.pitch + (wdense ? wcol : 0)) * kHeavyRec);
  // tiles T0 .. T0 + N - 1 of the wave's share into b_hi/b_lo[0 .. N - 1]
  auto load_tiles = [&](const h16x8 *sb, int T0, int N, int bs = 0) {
#pragma unroll
    for (int tt = 0; tt < N; ++tt) {
      b_hi[bs + tt] = sb[(T0 + tt) * 128 + lane];
      if (!HALF) b_lo[bs + tt] = sb[(T0 + tt) * 128 + 64 + lane];
    }
  };
  auto load_half = [&](const h16x8 *sb, int h) { load_tiles(sb, h * kHalf, kHalf); };
  // lane l holds rows 4(l/16) + i of item 16 tt + l%16
  int *const dbase = acc + (4 * (lane >> 4)) * Lp + wcol + (lane & 15);
  // products of tiles T0 .. T0 + N - 1 (add: a further block, summed into
  // the first block's values)
  auto mfma_tiles = [&](int T0, int N, bool add, int bs = 0) {
    if (!wdense) return;
#pragma unroll
    for (int tt = 0; tt < N; ++tt) {
      const int T = T0 + tt;
#pragma unroll
      for (int gi = 0; gi < kGroups; ++gi) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const f32x4 mn =
            __builtin_amdgcn_mfma_f32_16x16x32_f16(a_hi[gi], b_hi[bs + tt], z, 0, 0, 0);
        f32x4 cr;
        if (HALF) {  // item values in one fp16 (hi) each: query hi and lo times it
          cr = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_lo[gi], b_hi[bs + tt], z, 0, 0, 0);
        } else {
          cr = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_hi[gi], b_lo[bs + tt], z, 0, 0, 0);
          cr = __builtin_amdgcn_mfma_f32_16x16x32_f16(a_lo[gi], b_hi[bs + tt], cr, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int v = round_fix((mn[i] + cr[i] * (1.0f / kLoScale)) * kDenseToFix);
          if (gi == 0) dbase[i * Lp + 16 * T] = add ? dbase[i * Lp + 16 * T] + v : v;
          else dpend[T][i] = add ? dpend[T][i] + v : v;
        }
      }
    }
  };
  auto mfma_half = [&](int h, bool add) { mfma_tiles(h * kHalf, kHalf, add); };
  // The A tiles of both groups (4 KiB) are loaded once per workgroup by the
  // first 256 threads and shared through LDS (the segment table's space,
  // unused until the sparse part), not loaded by every wave.
  static_assert(kGroups * kTileHalves * 2 <= (kSegMax + kSegPad) * 4, "A tiles fit the staging");
  h16x8 *const astage = reinterpret_cast<h16x8 *>(s_spos);
  h16x8 aq;
  if (DENSE && t < kGroups * 128) {
    const int gi = t >> 7;
    aq = reinterpret_cast<const h16x8 *>(
        a.qh + (grp0 + (gi < ng ? gi : 0)) * (int64_t)a.qh_gstride)[t & 127];
  }
  if (DENSE) load_half(st, 0);
  __builtin_amdgcn_sched_barrier(0);
  if (DENSE) {
    if (t < kGroups * 128) astage[t] = aq;
    __syncthreads();
#pragma unroll
    for (int gi = 0; gi < kGroups; ++gi) {
      a_hi[gi] = astage[gi * 128 + lane];
      a_lo[gi] = astage[gi * 128 + 64 + lane];
    }
  }
  fetch_ranges(r0);
  fetch_ranges(r1);
  // Load order matters: the vector-memory counter drains in issue order.
  // The range lookups go out as soon as the entries are in (issued first,
  // they have mostly arrived by the staging barrier), after the first
  // half's slab tiles, so the first half's products do not wait for them;
  // the second half's products wait for its tiles, issued after the
  // lookups, by which time the lookups (random, often an L2 miss) have
  // mostly returned.
  if (DENSE) {
    mfma_half(0, false);
  } else {
    int4 *acc4 = reinterpret_cast<int4 *>(acc);
    for (int k = t; k < kRows * Lp / 4; k += NT) acc4[k] = make_int4(0, 0, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  if (DENSE) load_half(st, 1);
  __builtin_amdgcn_sched_barrier(0);
  if (DENSE) mfma_half(1, false);
  __builtin_amdgcn_sched_barrier(0);
  // Further blocks of 32 heavy dims (corpora with many dims held by a large
  // share of the items): tile by tile, each block's values rounded to fixed
  // point and added, so that every block keeps the error bound of one. Each
  // wave reads a block's A tiles itself (L1 hits after the first wave).
  auto load_block = [&](int b) {
#pragma unroll
    for (int gi = 0; gi < kGroups; ++gi) {
      const h16x8 *qb = reinterpret_cast<const h16x8 *>(
          a.qh + (grp0 + (gi < ng ? gi : 0)) * (int64_t)a.qh_gstride + b * kTileHalves);
      a_hi[gi] = qb[lane];
      a_lo[gi] = qb[64 + lane];
    }
    load_tiles(st + b * (a.slab_bstride / 8), 0, 1);
  };
  Desc cur, nxt;  // first batch of this group and of the next
  finish_ranges(r0, cur);
  finish_ranges(r1, nxt);
  // (a further block goes one tile at a time, the next tile's loads in flight
  // during this tile's products: two tiles held, not four)
  for (int b = 1; DENSE && b < nblk; ++b) {
    load_block(b);
    const h16x8 *sb = st + b * (a.slab_bstride / 8);
#pragma unroll
    for (int T = 0; T < kTiles; ++T) {
      // the next tile's loads go out before this tile's products
      if (T + 1 < kTiles) load_tiles(sb, T + 1, 1, (T + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
      mfma_tiles(T, 1, true, T & 1);
    }
  }
  // accumulators initialised before any sparse update: the first batch's scan
  // has a barrier (after every wave's part of the initial values above) and the
  // walk follows it; a first group with no light entries takes one here
  if (ge[0] == ge[1]) __syncthreads();

  const uint2 *__restrict__ ppost = a.post + cb0;
  const uint32_t *__restrict__ ppost4 = HALF ? a.post4 + cb0 : nullptr;
  const int64_t col0 = ib - g.chunk_begin(a.chunk);
  const bool v4 = vec4 && (col0 % 4 == 0);
  const bool full = v4 && slen == kSliceMax;
  // per-slice partial row sums only when row sums are asked for
  double *rsum = a.row_sums == nullptr ? nullptr : (g.n_sub == 1 ? a.row_sums : a.rs_part);
  int scan_par = 0;
  for (int gi = 0; gi < ng; ++gi) {
    const int64_t q0 = (grp0 + gi) * kRows;
    // the group's initial values into the accumulators: right after its first
    // batch's scan, whose barrier follows every wave's part of the previous
    // group's epilogue (a group with no light entries has no scan: barriers of
    // its own)
    auto init_acc = [&]() {
      if (DENSE) {
        if (wdense) {
#pragma unroll
          for (int tt = 0; tt < kTiles; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) dbase[i * Lp + 16 * tt] = dpend[tt][i];
        }
      } else {
        int4 *acc4 = reinterpret_cast<int4 *>(acc);
        for (int k = t; k < kRows * Lp / 4; k += NT) acc4[k] = make_int4(0, 0, 0, 0);
      }
    };
    if (gi > 0 && ge[gi] == ge[gi + 1]) {
      __syncthreads();
      init_acc();
      __syncthreads();
    }

    // ---- sparse part: the rows' light entries, batch by batch ----
    const int32_t e1 = ge[gi + 1];
    for (int32_t eb = ge[gi]; eb < e1; eb += kBatch) {
      // this batch's lists: the group's first batch was fetched at the start
      Desc c;
      if (eb == ge[gi]) {
        c = cur;
      } else {
        Raw r;
        const int32_t ee = batch_end(eb, e1);
        fetch_entries(r, eb, ee);
        fetch_ranges(r);
        finish_ranges(r, c);
      }
      int32_t nseg[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) nseg[i] = (c.L[i] + kSeg - 1) / kSeg;
      int32_t total;
      // (a barrier inside). Consecutive scans alternate between two buffers: a
      // batch with no segments has no barrier after its scan, so without them
      // a fast wave's next scan could overwrite totals a slow wave still reads.
      const int32_t pend = block_incl_scan_1b<NT>(nseg[0] + nseg[1], ws[scan_par], &total);
      scan_par ^= 1;
      if (gi > 0 && eb == ge[gi]) {
        init_acc();
        // (with no segments no round barrier follows: one before the epilogue)
        if (total == 0) __syncthreads();
      }
      const int32_t sp[2] = {pend - nseg[0] - nseg[1], pend - nseg[1]};
      for (int32_t r0 = 0; r0 < total; r0 += kSegMax) {
        // the segments of this round that belong to this thread's lists
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int32_t sb0 = sp[i] > r0 ? sp[i] : r0;
          const int32_t se = sp[i] + nseg[i] < r0 + kSegMax ? sp[i] + nseg[i] : r0 + kSegMax;
          for (int32_t sg = sb0; sg < se; ++sg) {
            const int32_t j0 = (sg - sp[i]) * kSeg;
            const int32_t n = c.L[i] - j0 < kSeg ? c.L[i] - j0 : kSeg;
            s_spos[sg - r0] = (uint32_t)(c.s[i] + j0);
            s_sqv[sg - r0] = __float_as_uint(c.qv[i]);
            s_smeta[sg - r0] = (uint32_t)n | ((uint32_t)(c.row[i] * Lp) << 7);  // byte offset << 5
          }
        }
        const int32_t nr = total - r0 < kSegMax ? total - r0 : kSegMax;
        for (int k = t; k < kSegPad; k += NT) s_smeta[nr + k] = 0u;
        __syncthreads();
        // Wave w takes segment groups w, w + NW, ...; lanes LPS i .. LPS i + LPS - 1
        // take segment i of a group (SPI segments), PPL postings per lane with
        // one 16-byte load, U groups per step.
        const int32_t jl = PPL * (lane % LPS);
        for (int32_t k0 = wv; SPI * k0 < nr; k0 += NW * U) {
          uint32_t pos[U];
          uint32_t aoff[U];
          float qv[U];
          int32_t nn[U];  // postings of the segment from this lane's first on
#pragma unroll
          for (int u = 0; u < U; ++u) {
            // entries past nr are padding (no postings)
            const int32_t sg = SPI * (k0 + NW * u) + lane / LPS;
            const uint32_t meta = s_smeta[sg];
            const uint32_t sp0 = s_spos[sg];
            nn[u] = (int32_t)(meta & 31u) - jl;
            pos[u] = nn[u] > 0 ? sp0 + jl : 0u;
            aoff[u] = meta >> 5;
            qv[u] = __uint_as_float(s_sqv[sg]);
          }
          // (the posting arrays hold padding entries past their ends, so a
          // lane's last postings stay readable at the end of an array)
          u32x4 pe[U];
#pragma unroll
          for (int u = 0; u < U; ++u)
            pe[u] = HALF ? ld_quad4(ppost4, pos[u] * 4u) : ld_pair(ppost, pos[u] * 8u);
          // all U loads are in flight before the first is waited on
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int u = 0; u < U; ++u) {
            char *const rbase = reinterpret_cast<char *>(acc) + aoff[u];
            if (HALF) {
              // (item | fp16(2^15 w) << 16) per posting
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                const uint32_t x = pe[u][k];
                const uint32_t it = x & 0xFFFFu;
                const float w = (float)__builtin_bit_cast(_Float16, (uint16_t)(x >> 16)) *
                                (1.0f / kHeavyScale);
                int *const p = nn[u] > k && it < (uint32_t)slen
                                   ? reinterpret_cast<int *>(rbase + 4 * it)
                                   : L.sink + lane;
                atomicAdd(p, round_fix(qv[u] * w));
              }
            } else {
              // (no bound check on the item: every posting the prepare writes,
              // the zero padding included, holds a slice-local id below the
              // slice size S <= Lp, so the address stays in acc[row][0, Lp)).
              // No branches either: a lane whose posting lies past its
              // segment's end adds to a slot of its own outside the
              // accumulators (distinct per lane, so no two lanes' dummy adds
              // meet at one address), which nothing reads.
              int *const p0 =
                  nn[u] > 0 ? reinterpret_cast<int *>(rbase + 4 * pe[u].x) : L.sink + lane;
              int *const p1 =
                  nn[u] > 1 ? reinterpret_cast<int *>(rbase + 4 * pe[u].z) : L.sink + lane;
              atomicAdd(p0, round_fix(qv[u] * __uint_as_float(pe[u].y)));
              atomicAdd(p1, round_fix(qv[u] * __uint_as_float(pe[u].w)));
            }
          }
        }
        __syncthreads();
      }
    }
    cur = nxt;

    if (MODE == kOutThreshold) {
      // ---- epilogue: the group's scores >= threshold as hits ----
      // Wave w counts rows w, w + NW, ... (and sums all their scores for the
      // row sums); each lane marks which of its (at most 16) scores of a row
      // are hits in a bit mask. One atomic per group reserves the group's
      // range of the hit buffer, laid out wave by wave, row by row, lane by
      // lane; then each lane writes its marked hits, reading only their
      // accumulators back.
      constexpr int RW = kRows / NW;
      static_assert(kSliceMax / 64 <= 32, "a lane's scores of a row fit a 32-bit mask");
      int cnt[RW], incl[RW], tot[RW];
      uint32_t hmask[RW];
      int wtot = 0;
#pragma unroll
      for (int rr = 0; rr < RW; ++rr) {
        const int r = wv + NW * rr;
        const int64_t q = q0 + r;
        const int4 *arow = reinterpret_cast<const int4 *>(acc + r * Lp);
        double rs = 0.0;
        uint32_t m = 0;
        if (q < a.n_q) {
          // score j0 + u of the lane is bit 4 step + u (j0 = 4 lane + 256 step)
          for (int j0 = 4 * lane; j0 < slen; j0 += 256) {
            const int4 x = arow[j0 >> 2];
            const int xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int u = 0; u < 4; ++u)
              if (j0 + u < slen) {
                const float v = (float)xs[u] * kFixInv;
                m |= (v >= a.threshold ? 1u : 0u) << (4 * (j0 >> 8) + u);
                rs += (double)v;
              }
          }
        }
        hmask[rr] = m;
        const int c = __builtin_popcount(m);
        cnt[rr] = c;
        incl[rr] = wave_incl_scan_dpp(c);
        tot[rr] = __builtin_amdgcn_readlane(incl[rr], 63);
        wtot += tot[rr];
        if (rsum != nullptr && q < a.n_q) {
          rs = wave_total_f64(rs);
          if (lane == 63) rsum[(g.n_sub == 1 ? 0 : (int64_t)ks * a.n_q) + q] = rs;
        }
      }
      if (lane == 0) s_wtot[wv] = wtot;
      __syncthreads();
      if (t == 0) {
        int sum = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) sum += s_wtot[w];
        s_hbase = sum > 0 ? atomicAdd(a.hit_count, (unsigned long long)sum) : 0ull;
      }
      __syncthreads();
      unsigned long long k0 = s_hbase;
      for (int w = 0; w < wv; ++w) k0 += (unsigned long long)s_wtot[w];
#pragma unroll
      for (int rr = 0; rr < RW; ++rr) {
        if (tot[rr] > 0) {
          const int r = wv + NW * rr;
          const int32_t q = (int32_t)(q0 + r);
          unsigned long long k = k0 + (unsigned long long)(incl[rr] - cnt[rr]);
          // the marked scores in increasing item order
          for (uint32_t m = hmask[rr]; m != 0u; m &= m - 1u) {
            const int b = __builtin_ctz(m);
            const int j = 4 * lane + 256 * (b >> 2) + (b & 3);
            const float v = (float)acc[r * Lp + j] * kFixInv;
            if (k < (unsigned long long)a.hit_cap)
              a.hits[k] = make_int3(q, (int32_t)(ib + j), __float_as_int(v));
            ++k;
          }
          k0 += (unsigned long long)tot[rr];
        }
      }
      continue;
    }

    // ---- epilogue: wave w writes rows w, w + NW, ... of the group ----
#pragma unroll
    for (int rr = 0; rr < kRows / NW; ++rr) {
      const int r = wv + NW * rr;
      const int64_t q = q0 + r;
      if (q >= a.n_q) break;
      const int4 *arow = reinterpret_cast<const int4 *>(acc + r * Lp);
      double rs = 0.0;
      if (HALF) {
        // fp16(fl32(acc) * 2^-30), 8-byte stores when aligned; the row sum is
        // of the fp16 values written
        uint16_t *hrow = a.out16 + q * a.ld + col0;
        for (int j0 = 4 * lane; j0 < slen; j0 += 256) {
          const int4 x = arow[j0 >> 2];
          const _Float16 h[4] = {(_Float16)((float)x.x * kFixInv), (_Float16)((float)x.y * kFixInv),
                                 (_Float16)((float)x.z * kFixInv), (_Float16)((float)x.w * kFixInv)};
          if (v4 && j0 + 3 < slen) {
            const u32x2 pk = {(uint32_t)__builtin_bit_cast(uint16_t, h[0]) |
                                  ((uint32_t)__builtin_bit_cast(uint16_t, h[1]) << 16),
                              (uint32_t)__builtin_bit_cast(uint16_t, h[2]) |
                                  ((uint32_t)__builtin_bit_cast(uint16_t, h[3]) << 16)};
            __builtin_nontemporal_store(pk, reinterpret_cast<u32x2 *>(hrow + j0));
            rs += ((double)(float)h[0] + (double)(float)h[1]) +
                  ((double)(float)h[2] + (double)(float)h[3]);
          } else {
#pragma unroll
            for (int u = 0; u < 4; ++u)
              if (j0 + u < slen) {
                hrow[j0 + u] = __builtin_bit_cast(uint16_t, h[u]);
                rs += (double)(float)h[u];
              }
          }
        }
        if (rsum != nullptr) {
          rs = wave_total_f64(rs);
          if (lane == 63) rsum[(g.n_sub == 1 ? 0 : (int64_t)ks * a.n_q) + q] = rs;
        }
        continue;
      }
      float *orow = a.out + q * a.ld + col0;
      if (full) {
        // a whole slice with aligned rows (every slice but a corpus's last):
        // four 16-byte reads and stores per lane and no per-lane conditions
        int4 xs[kSliceMax / 256];
#pragma unroll
        for (int k = 0; k < kSliceMax / 256; ++k) xs[k] = arow[lane + 64 * k];
        float *const o = orow + 4 * lane;
        double fs = 0.0;
#pragma unroll
        for (int k = 0; k < kSliceMax / 256; ++k) {
          const int4 x = xs[k];
          const f32x4 v = {(float)x.x * kFixInv, (float)x.y * kFixInv, (float)x.z * kFixInv,
                           (float)x.w * kFixInv};
          __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(o + 256 * k));
          const double s4 = ((double)v[0] + (double)v[1]) + ((double)v[2] + (double)v[3]);
          fs = k == 0 ? s4 : fs + s4;
          // one store per block of conversions: a burst of stores stalls the
          // other workgroup's loads
          __builtin_amdgcn_sched_barrier(0);
        }
        rs = fs;
        if (rsum != nullptr) {
          rs = wave_total_f64(rs);
          if (lane == 63) rsum[(g.n_sub == 1 ? 0 : (int64_t)ks * a.n_q) + q] = rs;
        }
        continue;
      }
      // the row's (at most four) 16-byte accumulator reads go out together
      int4 xs[kSliceMax / 256];
#pragma unroll
      for (int k = 0; k < kSliceMax / 256; ++k)
        if (4 * lane + 256 * k < slen) xs[k] = arow[lane + 64 * k];
#pragma unroll
      for (int k = 0; k < kSliceMax / 256; ++k) {
        const int j0 = 4 * lane + 256 * k;
        if (j0 >= slen) continue;
        const int4 x = xs[k];
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
      if (rsum != nullptr) {
        rs = wave_total_f64(rs);
        if (lane == 63) rsum[(g.n_sub == 1 ? 0 : (int64_t)ks * a.n_q) + q] = rs;
      }
    }
  }
}

template <bool DENSE, int MODE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) void score_kernel(
    const ScoreArgs a, int vec4) {
  extern __shared__ int acc[];
  __shared__ uint32_t s_spos[kSegMax + kSegPad], s_sqv[kSegMax + kSegPad],
      s_smeta[kSegMax + kSegPad];
  __shared__ int32_t ws[2][NW];
  __shared__ int32_t s_wtot[NW];
  __shared__ unsigned long long s_hbase;
  __shared__ int s_sink[64];
  const ScoreLds L{acc, s_spos, s_sqv, s_smeta, ws, s_wtot, &s_hbase, s_sink};
  // heavy-dim blocks in use (the slab and the query tiles hold a.heavy_blocks);
  // a corpus with no heavy dims takes the path without the dense part. The
  // choice is uniform across the workgroup.
  const int nh = DENSE ? a.heavy[kHeavyMax] : 0;
  int nblk = heavy_blocks(nh);
  nblk = nblk < a.heavy_blocks ? nblk : a.heavy_blocks;
  if (DENSE && nblk == 0) score_body<false, MODE>(a, vec4, L, 0);
  else score_body<DENSE, MODE>(a, vec4, L, nblk);
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
  return (size_t)kRows * acc_pitch(S) * sizeof(int) + (kSegMax + kSegPad) * 12 + 2 * NW * 4 + 8 + 64 * 4;
}

template <bool DENSE, int MODE>
static hipError_t launch_t(const ScoreArgs &a, hipStream_t s) {
  constexpr bool HALF = MODE == kOutHalf;
  const size_t dyn = (size_t)kRows * acc_pitch(a.g.S) * sizeof(int);
  auto kern = score_kernel<DENSE, MODE>;
  // dynamic LDS above 64 KiB needs an explicit opt-in per kernel, made once
  // per device (and again if a later corpus needs more); callers on several
  // threads may race to make it, which is harmless
  constexpr int kMaxDevices = 64;
  static std::atomic<size_t> opted[kMaxDevices];
  if (dyn > 65536) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    size_t cur = opted[dev].load(std::memory_order_relaxed);
    if (dyn > cur) {
      e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
      if (e != hipSuccess) return e;
      while (cur < dyn && !opted[dev].compare_exchange_weak(cur, dyn, std::memory_order_relaxed)) {
      }
    }
  }
  // wide stores need the row pitch and base aligned: 16 bytes (fp32), 8 (fp16)
  const uintptr_t base = HALF ? reinterpret_cast<uintptr_t>(a.out16)
                              : reinterpret_cast<uintptr_t>(a.out);
  const int vec4 = (a.ld % 4 == 0) && ((base & (HALF ? 7 : 15)) == 0);
  const int64_t pairs = (a.n_groups + kGroups - 1) / kGroups;
  hipLaunchKernelGGL(kern, dim3((unsigned)(pairs * a.g.n_sub)), dim3(NT), dyn, s, a, vec4);
  return hipGetLastError();
}

hipError_t launch_score(const ScoreArgs &a, hipStream_t s) {
  if (a.n_groups == 0) return hipSuccess;
  hipError_t e;
  // the mode is explicit: a threshold pass may count without a hit buffer
  // (capacity 0, hits null), which must not select a scoring mode
  switch (a.mode) {
    case kModeThreshold:
      if (a.hit_count == nullptr || (a.hit_cap > 0 && a.hits == nullptr))
        return hipErrorInvalidValue;
      e = a.dense ? launch_t<true, kOutThreshold>(a, s) : launch_t<false, kOutThreshold>(a, s);
      break;
    case kModeHalf:
      if (a.out16 == nullptr || a.post4 == nullptr) return hipErrorInvalidValue;
      e = a.dense ? launch_t<true, kOutHalf>(a, s) : launch_t<false, kOutHalf>(a, s);
      break;
    case kModeExact:
      if (a.out == nullptr) return hipErrorInvalidValue;
      e = a.dense ? launch_t<true, kOutExact>(a, s) : launch_t<false, kOutExact>(a, s);
      break;
    default:
      return hipErrorInvalidValue;
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
