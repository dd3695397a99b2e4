// sps_api.hip -- the C ABI of include/sps.h: argument checks, workspace
// layout, handles and stream-ordered launches. Host code only; the kernels
// live in sps_prepare.hip and sps_score.hip.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>

#include "sps.h"
#include "sps_internal.h"

// Device scratch of sps_cosine_chunk_static: the per-slice partial row sums,
// held by the library on every GPU it runs on until the process ends. Host
// code must never use this name as a device address (in host code it is a
// host-side stand-in): the device address comes from hipGetSymbolAddress,
// once per device (scratch_address below).
constexpr int64_t kStaticScratchDoubles = 1 << 19;  // 4 MiB
static __device__ __align__(256) double scratch[kStaticScratchDoubles];

namespace {

thread_local char g_err[512] = "";

sps_status fail(sps_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

sps_status hip_fail(hipError_t e, const char *where) {
  return fail(SPS_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr int64_t kI32Max = 2147483647ll;
constexpr size_t kAlign = 256;
constexpr int32_t kMaxChunk = 1 << 20;

size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

// Byte layout builder: adds 256-aligned regions, detects overflow.
struct Layout {
  size_t off = 0;
  bool overflow = false;
  size_t add(uint64_t count, uint64_t elem) {
    const size_t at = off;
    if (elem != 0 && count > (UINT64_MAX / 4) / elem) {
      overflow = true;
      return at;
    }
    const uint64_t bytes = count * elem;
    const size_t next = align_up(off + (size_t)bytes);
    if (next < off) overflow = true;
    off = next;
    return at;
  }
};

sps_status check_csr_shape(const sps_csr *m, const char *what) {
  if (!m) return fail(SPS_ERR_INVALID_ARGUMENT, "%s: NULL CSR", what);
  if (m->n_rows < 0 || m->n_cols <= 0 || m->nnz < 0)
    return fail(SPS_ERR_INVALID_ARGUMENT, "%s: negative size or n_cols <= 0", what);
  if (m->n_rows >= kI32Max || m->n_cols >= kI32Max || m->nnz >= kI32Max)
    return fail(SPS_ERR_OVERFLOW, "%s: sizes must be below 2^31", what);
  if (!m->indptr) return fail(SPS_ERR_INVALID_ARGUMENT, "%s: NULL indptr", what);
  if (m->nnz > 0 && (!m->indices || !m->values))
    return fail(SPS_ERR_INVALID_ARGUMENT, "%s: NULL indices or values", what);
  return SPS_OK;
}

// The device address of `scratch` on the current device, looked up on the
// first call on each device and kept (each GPU holds its own copy).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_addr[kMaxDevices];

sps_status scratch_address(double **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SPS_ERR_UNSUPPORTED, "device %d beyond the %d this library tracks", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_addr[dev] = p;
  }
  *out = static_cast<double *>(g_scratch_addr[dev]);
  return SPS_OK;
}

// The heavy-dim dense path is on for slices it supports unless SPS_DENSE=0.
bool dense_wanted(const sps::Geom &g) {
  if (!sps::dense_slice_ok(g.S)) return false;
  if (const char *env = getenv("SPS_DENSE")) return atoi(env) != 0;
  return true;
}

// Most heavy dims to take, kHeavyMax unless SPS_HEAVY_MAX (0..kHeavyMax) says
// otherwise (a tuning knob: results do not depend on it beyond rounding).
int32_t heavy_cap() {
  if (const char *env = getenv("SPS_HEAVY_MAX")) {
    const int v = atoi(env);
    if (v >= 0 && v <= sps::kHeavyMax) return v;
  }
  return sps::kHeavyMax;
}

// Gain a further heavy-dim block must bring (see heavy_rank_kernel):
// kHeavyBlockGain unless SPS_HEAVY_GAIN (>= 0) says otherwise (a tuning knob:
// results do not depend on it beyond rounding).
float heavy_gain() {
  if (const char *env = getenv("SPS_HEAVY_GAIN")) {
    const double v = atof(env);
    if (v >= 0.0 && v < 1e30) return (float)v;
  }
  return sps::kHeavyBlockGain;
}

template <typename T>
T *at(void *base, size_t off) {
  return reinterpret_cast<T *>(reinterpret_cast<char *>(base) + off);
}

struct ItemsLayout {
  size_t inv, dinfo, dtab, post, sbase, heavy, slab, persistent;
  size_t flags, norm64, skey0, skey1, spay, gdf, hsel, scratch;
  bool overflow;
};

// Halves from one heavy-dim block's slab to the next's.
int64_t slab_block_stride(const sps::Geom &g) {
  return g.num_slices() * (int64_t)sps::kHeavyRec * sps::slab_pitch(g.S);
}

ItemsLayout items_layout(const sps::Geom &g, int64_t dim, int64_t nnz, bool dense, int32_t cap) {
  const int64_t ns = g.num_slices();
  ItemsLayout L{};
  Layout p;
  L.inv = p.add(g.n_items, 4);
  L.dinfo = p.add(ns + 1, 16);
  // a slice's table has max(1, 2 * distinct dims) buckets and distinct <= its nnz
  L.dtab = p.add(sps::kBucketsPerDim * (uint64_t)nnz + (uint64_t)ns, 16);
  L.post = p.add(nnz + sps::kPostPad, 8);
  L.sbase = p.add(ns + 1, 4);
  L.heavy = p.add(sps::kHeavyMax + 1, 4);
  L.slab = p.add(dense ? (uint64_t)sps::heavy_blocks(cap) * (uint64_t)slab_block_stride(g) : 0, 2);
  L.persistent = p.off;
  Layout s;
  L.flags = s.add(sps::kFlagsInts, 4);
  L.norm64 = s.add(g.n_items, 8);
  L.skey0 = s.add(nnz, 4);
  L.skey1 = s.add(nnz, 4);
  L.spay = s.add(nnz, 8);
  L.gdf = s.add(dense ? (uint64_t)sps::kGdfStripes * (uint64_t)dim : 0, 4);
  L.hsel = s.add(dense ? sps::kHeavySelInts : 0, 4);
  L.scratch = s.off;
  L.overflow = p.overflow || s.overflow;
  return L;
}

struct QueriesLayout {
  size_t flags, inv, norm64, lptr, lrec, qh, rspart, total;
  bool overflow;
};

QueriesLayout queries_layout(int64_t n, int64_t nnz, int32_t n_sub, bool dense, int32_t qh_gstride) {
  const int64_t ng = (n + sps::kRows - 1) / sps::kRows;
  QueriesLayout L{};
  Layout p;
  L.flags = p.add(sps::kFlagsInts, 4);
  L.inv = p.add(n, 4);
  L.norm64 = p.add(n, 8);
  L.lptr = p.add(n + 1, 4);
  // at least one light entry each: the score kernel may read entry 0 of an
  // empty batch (and ignores it)
  L.lrec = p.add(nnz > 0 ? nnz : 1, 12);
  L.qh = p.add(dense ? (uint64_t)ng * (uint64_t)qh_gstride : 0, 2);
  L.rspart = p.add(n_sub > 1 ? (uint64_t)n_sub * (uint64_t)n : 0, 8);
  L.total = p.off;
  L.overflow = p.overflow;
  return L;
}

}  // namespace

struct sps_items {
  sps::Geom g;
  int64_t dim, nnz;
  int device;
  bool dense;
  int32_t pitch;         // slab row pitch (items), dense only
  int32_t heavy_blocks;  // heavy-dim blocks the slab holds (dense only)
  int64_t slab_bstride;  // halves from one block's slab to the next's
  float *inv_norm;
  int4 *dinfo;
  uint4 *dtab;
  uint2 *post;
  int32_t *slice_base;
  int32_t *heavy;
  uint16_t *slab;
  uint32_t *post4;  // reduced-precision postings (null until sps_items_enable_half)
};

struct sps_queries {
  int64_t n_rows, dim, nnz;
  int32_t n_groups;
  int device;
  bool dense;
  const sps_items *items;  // the corpus the queries were prepared for
  float *inv_norm;
  int32_t *lptr;
  uint3 *lrec;
  uint16_t *qh;
  int32_t qh_gstride;  // halves per row group in qh
  double *rs_part;
};

namespace {
// halves per 16-row group of a query batch's heavy-dim tiles: one tile per
// block the items' slab holds
int32_t qh_group_stride(const sps_items *items) { return items->heavy_blocks * sps::kTileHalves; }
}  // namespace

extern "C" {

const char *sps_status_string(sps_status s) {
  switch (s) {
    case SPS_OK: return "ok";
    case SPS_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SPS_ERR_BAD_CSR: return "non-canonical CSR";
    case SPS_ERR_DIM_MISMATCH: return "query and item dimensions differ";
    case SPS_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case SPS_ERR_CHUNK_RANGE: return "chunk index out of range";
    case SPS_ERR_OVERFLOW: return "size overflow";
    case SPS_ERR_HIP: return "HIP runtime error";
    case SPS_ERR_UNSUPPORTED: return "unsupported configuration";
  }
  return "unknown status";
}

const char *sps_last_error_message(void) { return g_err; }

sps_status sps_items_workspace_size(int64_t n_items, int64_t dim, int64_t nnz,
                                    int32_t chunk_size, size_t *persistent_bytes,
                                    size_t *scratch_bytes) {
  if (!persistent_bytes || !scratch_bytes)
    return fail(SPS_ERR_INVALID_ARGUMENT, "NULL output pointer");
  if (n_items < 0 || dim <= 0 || nnz < 0)
    return fail(SPS_ERR_INVALID_ARGUMENT, "negative size or dim <= 0");
  if (chunk_size < 1 || chunk_size > kMaxChunk)
    return fail(SPS_ERR_INVALID_ARGUMENT, "chunk_size must be in [1, %d]", kMaxChunk);
  if (n_items >= kI32Max || dim >= kI32Max || nnz >= kI32Max)
    return fail(SPS_ERR_OVERFLOW, "sizes must be below 2^31");
  if (nnz >= (1ll << 29) - 64)
    return fail(SPS_ERR_OVERFLOW, "item nnz must be below 2^29 - 64 (32-bit posting byte offsets)");
  const sps::Geom g = sps::make_geom(n_items, chunk_size);
  const ItemsLayout L = items_layout(g, dim, nnz, dense_wanted(g), heavy_cap());
  if (L.overflow) return fail(SPS_ERR_OVERFLOW, "workspace byte count overflows");
  *persistent_bytes = L.persistent;
  *scratch_bytes = L.scratch;
  return SPS_OK;
}

sps_status sps_prepare(const sps_csr *items, int32_t chunk_size, void *persistent,
                       size_t persistent_bytes, void *scratch, size_t scratch_bytes,
                       void *stream, sps_items **out) {
  if (!out) return fail(SPS_ERR_INVALID_ARGUMENT, "NULL output handle pointer");
  *out = nullptr;
  sps_status st = check_csr_shape(items, "items");
  if (st != SPS_OK) return st;
  size_t need_p = 0, need_s = 0;
  st = sps_items_workspace_size(items->n_rows, items->n_cols, items->nnz, chunk_size, &need_p,
                                &need_s);
  if (st != SPS_OK) return st;
  if (!persistent || !scratch) return fail(SPS_ERR_INVALID_ARGUMENT, "NULL workspace");
  if (persistent_bytes < need_p || scratch_bytes < need_s)
    return fail(SPS_ERR_WORKSPACE_TOO_SMALL,
                "need %zu persistent and %zu scratch bytes, got %zu and %zu", need_p, need_s,
                persistent_bytes, scratch_bytes);
  if ((reinterpret_cast<uintptr_t>(persistent) | reinterpret_cast<uintptr_t>(scratch)) & 255)
    return fail(SPS_ERR_INVALID_ARGUMENT, "workspaces must be 256-byte aligned");
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(SPS_ERR_HIP, "no HIP device");

  const sps::Geom g = sps::make_geom(items->n_rows, chunk_size);
  const bool dense = dense_wanted(g);
  const int32_t cap = heavy_cap();
  const ItemsLayout L = items_layout(g, items->n_cols, items->nnz, dense, cap);
  sps::ItemsDev d{};
  d.g = g;
  d.dim = items->n_cols;
  d.nnz = items->nnz;
  d.dense = dense;
  d.heavy_cap = cap;
  d.slab_bstride = slab_block_stride(g);
  d.heavy_gain = heavy_gain();
  d.indptr = items->indptr;
  d.indices = items->indices;
  d.values = items->values;
  d.inv_norm = at<float>(persistent, L.inv);
  d.dinfo = at<int4>(persistent, L.dinfo);
  d.dtab = at<uint4>(persistent, L.dtab);
  d.post = at<uint2>(persistent, L.post);
  d.slice_base = at<int32_t>(persistent, L.sbase);
  d.heavy = at<int32_t>(persistent, L.heavy);
  d.slab = dense ? at<uint16_t>(persistent, L.slab) : nullptr;
  d.flags = at<int32_t>(scratch, L.flags);
  d.norm64 = at<double>(scratch, L.norm64);
  d.skey[0] = at<int32_t>(scratch, L.skey0);
  d.skey[1] = at<int32_t>(scratch, L.skey1);
  d.spay = at<uint2>(scratch, L.spay);
  d.gdf = dense ? at<int32_t>(scratch, L.gdf) : nullptr;
  d.hsel = dense ? at<int32_t>(scratch, L.hsel) : nullptr;

  sps_items *h = new (std::nothrow) sps_items;
  if (!h) return fail(SPS_ERR_INVALID_ARGUMENT, "out of host memory");
  hipError_t e = sps::launch_prepare_items(d, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    delete h;
    return hip_fail(e, "sps_prepare");
  }
  h->g = g;
  h->dim = d.dim;
  h->nnz = d.nnz;
  h->device = dev;
  h->dense = dense;
  h->pitch = dense ? sps::slab_pitch(g.S) : 0;
  h->heavy_blocks = dense ? sps::heavy_blocks(cap) : 0;
  h->slab_bstride = d.slab_bstride;
  h->inv_norm = d.inv_norm;
  h->dinfo = d.dinfo;
  h->dtab = d.dtab;
  h->post = d.post;
  h->slice_base = d.slice_base;
  h->heavy = d.heavy;
  h->slab = d.slab;
  h->post4 = nullptr;
  *out = h;
  return SPS_OK;
}

sps_status sps_items_info(const sps_items *h, int64_t *n_items, int64_t *dim, int64_t *nnz,
                          int32_t *chunk_size, int32_t *num_chunks) {
  if (!h) return fail(SPS_ERR_INVALID_ARGUMENT, "NULL handle");
  if (n_items) *n_items = h->g.n_items;
  if (dim) *dim = h->dim;
  if (nnz) *nnz = h->nnz;
  if (chunk_size) *chunk_size = h->g.C;
  if (num_chunks) *num_chunks = h->g.num_chunks;
  return SPS_OK;
}

sps_status sps_items_slices(const sps_items *h, int32_t *slice_size, int32_t *slices_per_chunk,
                            int64_t *num_slices) {
  if (!h) return fail(SPS_ERR_INVALID_ARGUMENT, "NULL handle");
  if (slice_size) *slice_size = h->g.S;
  if (slices_per_chunk) *slices_per_chunk = h->g.n_sub;
  if (num_slices) *num_slices = h->g.num_slices();
  return SPS_OK;
}

sps_status sps_items_slice_view(const sps_items *h, int64_t slice, void *stream,
                                sps_slice_view *view) {
  if (!h || !view) return fail(SPS_ERR_INVALID_ARGUMENT, "NULL handle or view");
  if (slice < 0 || slice >= h->g.num_slices())
    return fail(SPS_ERR_CHUNK_RANGE, "slice %lld outside [0, %lld)", (long long)slice,
                (long long)h->g.num_slices());
  hipError_t e = hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "sps_items_slice_view");
  int32_t be[2];
  e = hipMemcpy(be, h->slice_base + slice, sizeof be, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "sps_items_slice_view");
  view->item_begin = h->g.slice_begin(slice);
  view->slice_len = (int32_t)(h->g.slice_end(slice) - view->item_begin);
  view->slice_nnz = be[1] - be[0];
  view->post = reinterpret_cast<const sps_posting *>(h->post + be[0]);
  view->item_inv_norm = h->inv_norm + view->item_begin;
  return SPS_OK;
}

sps_status sps_items_slice_col_ptr(const sps_items *h, int64_t slice, int32_t *col_ptr,
                                   int32_t *status, void *stream) {
  if (!h || !col_ptr) return fail(SPS_ERR_INVALID_ARGUMENT, "NULL handle or col_ptr");
  if (slice < 0 || slice >= h->g.num_slices())
    return fail(SPS_ERR_CHUNK_RANGE, "slice %lld outside [0, %lld)", (long long)slice,
                (long long)h->g.num_slices());
  const hipError_t e =
      sps::launch_expand_col_ptr(h->dim, h->dinfo, h->dtab, h->slice_base, slice, col_ptr, status,
                                 reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "sps_items_slice_col_ptr");
  return SPS_OK;
}

sps_status sps_items_heavy_dims(const sps_items *h, void *stream, int32_t *dims,
                                int32_t capacity, int32_t *count) {
  if (!h || !count) return fail(SPS_ERR_INVALID_ARGUMENT, "NULL argument");
  hipError_t e = hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "sps_items_heavy_dims");
  int32_t buf[sps::kHeavyMax + 1];
  e = hipMemcpy(buf, h->heavy, sizeof buf, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "sps_items_heavy_dims");
  const int32_t m = h->dense ? buf[sps::kHeavyMax] : 0;
  *count = m;
  if (dims)
    for (int32_t i = 0; i < m && i < capacity; ++i) dims[i] = buf[i];
  return SPS_OK;
}

void sps_items_destroy(sps_items *h) { delete h; }

sps_status sps_queries_workspace_size(const sps_items *items, int64_t n_rows, int64_t dim,
                                      int64_t nnz, size_t *bytes) {
  if (!items || !bytes) return fail(SPS_ERR_INVALID_ARGUMENT, "NULL argument");
  if (n_rows < 0 || dim <= 0 || nnz < 0)
    return fail(SPS_ERR_INVALID_ARGUMENT, "negative size or dim <= 0");
  if (n_rows >= kI32Max || dim >= kI32Max || nnz >= kI32Max)
    return fail(SPS_ERR_OVERFLOW, "sizes must be below 2^31");
  if (dim != items->dim)
    return fail(SPS_ERR_DIM_MISMATCH, "query dim %lld != item dim %lld", (long long)dim,
                (long long)items->dim);
  const QueriesLayout L =
      queries_layout(n_rows, nnz, items->g.n_sub, items->dense, qh_group_stride(items));
  if (L.overflow) return fail(SPS_ERR_OVERFLOW, "workspace byte count overflows");
  *bytes = L.total;
  return SPS_OK;
}

sps_status sps_prepare_queries(const sps_csr *queries, const sps_items *items, void *workspace,
                               size_t workspace_bytes, void *stream, sps_queries **out) {
  if (!out) return fail(SPS_ERR_INVALID_ARGUMENT, "NULL output handle pointer");
  *out = nullptr;
  sps_status st = check_csr_shape(queries, "queries");
  if (st != SPS_OK) return st;
  if (!items) return fail(SPS_ERR_INVALID_ARGUMENT, "NULL items handle");
  size_t need = 0;
  st = sps_queries_workspace_size(items, queries->n_rows, queries->n_cols, queries->nnz, &need);
  if (st != SPS_OK) return st;
  if (!workspace) return fail(SPS_ERR_INVALID_ARGUMENT, "NULL workspace");
  if (workspace_bytes < need)
    return fail(SPS_ERR_WORKSPACE_TOO_SMALL, "need %zu bytes, got %zu", need, workspace_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) & 255)
    return fail(SPS_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(SPS_ERR_HIP, "no HIP device");
  const bool dense = items->dense;
  const QueriesLayout L = queries_layout(queries->n_rows, queries->nnz, items->g.n_sub, dense,
                                         qh_group_stride(items));
  sps::QueriesDev d{};
  d.n_rows = queries->n_rows;
  d.dim = queries->n_cols;
  d.nnz = queries->nnz;
  d.n_groups = (int32_t)((queries->n_rows + sps::kRows - 1) / sps::kRows);
  d.dense = dense;
  d.indptr = queries->indptr;
  d.indices = queries->indices;
  d.values = queries->values;
  d.heavy = items->heavy;
  d.qh_gstride = qh_group_stride(items);
  d.flags = at<int32_t>(workspace, L.flags);
  d.inv_norm = at<float>(workspace, L.inv);
  d.norm64 = at<double>(workspace, L.norm64);
  d.lptr = at<int32_t>(workspace, L.lptr);
  d.lrec = at<uint3>(workspace, L.lrec);
  d.qh = dense ? at<uint16_t>(workspace, L.qh) : nullptr;
  sps_queries *h = new (std::nothrow) sps_queries;
  if (!h) return fail(SPS_ERR_INVALID_ARGUMENT, "out of host memory");
  hipError_t e = sps::launch_prepare_queries(d, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    delete h;
    return hip_fail(e, "sps_prepare_queries");
  }
  h->n_rows = d.n_rows;
  h->dim = d.dim;
  h->nnz = d.nnz;
  h->n_groups = d.n_groups;
  h->device = dev;
  h->dense = dense;
  h->items = items;
  h->inv_norm = d.inv_norm;
  h->lptr = d.lptr;
  h->lrec = d.lrec;
  h->qh = d.qh;
  h->qh_gstride = d.qh_gstride;
  h->rs_part = items->g.n_sub > 1 ? at<double>(workspace, L.rspart) : nullptr;
  *out = h;
  return SPS_OK;
}

sps_status sps_queries_inv_norms(const sps_queries *q, const float **inv_norm) {
  if (!q || !inv_norm) return fail(SPS_ERR_INVALID_ARGUMENT, "NULL argument");
  *inv_norm = q->inv_norm;
  return SPS_OK;
}

void sps_queries_destroy(sps_queries *q) { delete q; }

static sps_status check_score_args(const sps_queries *q, const sps_items *items, const void *out,
                                   int64_t ld_out) {
  if (!q || !items) return fail(SPS_ERR_INVALID_ARGUMENT, "NULL handle");
  if (q->items != items)
    return fail(SPS_ERR_INVALID_ARGUMENT, "queries were prepared for another item corpus");
  if (q->n_rows > 0 && !out) return fail(SPS_ERR_INVALID_ARGUMENT, "NULL output");
  const int64_t width = items->g.C < items->g.n_items ? items->g.C : items->g.n_items;
  if (ld_out < width)
    return fail(SPS_ERR_INVALID_ARGUMENT, "ld_out %lld below the chunk length %lld",
                (long long)ld_out, (long long)width);
  if (q->n_rows > 0 && (uint64_t)ld_out > (uint64_t)INT64_MAX / 4 / (uint64_t)q->n_rows)
    return fail(SPS_ERR_OVERFLOW, "n_rows * ld_out overflows");
  // one workgroup per (row group, slice) in a one-dimensional grid
  if ((int64_t)q->n_groups * items->g.n_sub > kI32Max)
    return fail(SPS_ERR_OVERFLOW, "%lld row groups x %d slices exceed the launch grid",
                (long long)q->n_groups, items->g.n_sub);
  return SPS_OK;
}

static sps_status score_one(const sps_queries *q, const sps_items *items, int32_t chunk,
                            sps::ScoreMode mode, float *out, uint16_t *out16, int64_t ld_out,
                            double *row_sums, hipStream_t s, const sps::ScoreArgs *extra = nullptr,
                            double *rs_part = nullptr) {
  sps::ScoreArgs a{};
  if (extra) a = *extra;
  a.mode = mode;
  a.g = items->g;
  a.dim = items->dim;
  a.n_q = q->n_rows;
  a.n_groups = q->n_groups;
  a.chunk = chunk;
  a.dense = q->dense && items->dense;
  a.lptr = q->lptr;
  a.lrec = q->lrec;
  a.qh = q->qh;
  a.qh_gstride = q->qh_gstride;
  a.dinfo = items->dinfo;
  a.dtab = items->dtab;
  a.post = items->post;
  a.post4 = items->post4;
  a.slice_base = items->slice_base;
  a.heavy = items->heavy;
  a.slab = items->slab;
  a.slab_bstride = items->slab_bstride;
  a.heavy_blocks = items->heavy_blocks;
  a.pitch = items->pitch;
  a.out = out;
  a.out16 = out16;
  a.ld = ld_out;
  a.rs_part = rs_part != nullptr ? rs_part : q->rs_part;
  a.row_sums = row_sums;
  const hipError_t e = sps::launch_score(a, s);
  if (e != hipSuccess) return hip_fail(e, "score kernel");
  return SPS_OK;
}

sps_status sps_cosine_chunk(const sps_queries *q, const sps_items *items, int32_t chunk,
                            float *out, int64_t ld_out, double *row_sums, void *stream) {
  sps_status st = check_score_args(q, items, out, ld_out);
  if (st != SPS_OK) return st;
  if (chunk < 0 || chunk >= items->g.num_chunks)
    return fail(SPS_ERR_CHUNK_RANGE, "chunk %d outside [0, %d)", chunk, items->g.num_chunks);
  return score_one(q, items, chunk, sps::kModeExact, out, nullptr, ld_out, row_sums,
                   reinterpret_cast<hipStream_t>(stream));
}

sps_status sps_cosine_chunk_static(const sps_queries *q, const sps_items *items, int32_t chunk,
                                   float *out, int64_t ld_out, double *row_sums, void *stream) {
  sps_status st = check_score_args(q, items, out, ld_out);
  if (st != SPS_OK) return st;
  if (chunk < 0 || chunk >= items->g.num_chunks)
    return fail(SPS_ERR_CHUNK_RANGE, "chunk %d outside [0, %d)", chunk, items->g.num_chunks);
  double *part = nullptr;
  if (row_sums != nullptr && items->g.n_sub > 1) {
    const int64_t need = (int64_t)items->g.n_sub * q->n_rows;
    if (need > kStaticScratchDoubles)
      return fail(SPS_ERR_UNSUPPORTED,
                  "row sums of %lld rows x %d slices need %lld doubles of scratch; the "
                  "library's static scratch holds %lld (use sps_cosine_chunk)",
                  (long long)q->n_rows, items->g.n_sub, (long long)need,
                  (long long)kStaticScratchDoubles);
    st = scratch_address(&part);
    if (st != SPS_OK) return st;
  }
  return score_one(q, items, chunk, sps::kModeExact, out, nullptr, ld_out, row_sums,
                   reinterpret_cast<hipStream_t>(stream), nullptr, part);
}

sps_status sps_cosine_chunk_threshold(const sps_queries *q, const sps_items *items, int32_t chunk,
                                      float threshold, sps_hit *hits, int64_t capacity,
                                      uint64_t *count, double *row_sums, void *stream) {
  if (!q || !items || !count) return fail(SPS_ERR_INVALID_ARGUMENT, "NULL argument");
  if (capacity < 0 || (capacity > 0 && !hits))
    return fail(SPS_ERR_INVALID_ARGUMENT, "negative capacity or NULL hits");
  if (threshold != threshold) return fail(SPS_ERR_INVALID_ARGUMENT, "threshold is NaN");
  const int64_t width = items->g.C < items->g.n_items ? items->g.C : items->g.n_items;
  sps_status st = check_score_args(q, items, count, width);
  if (st != SPS_OK) return st;
  if (chunk < 0 || chunk >= items->g.num_chunks)
    return fail(SPS_ERR_CHUNK_RANGE, "chunk %d outside [0, %d)", chunk, items->g.num_chunks);
  static_assert(sizeof(sps_hit) == 12, "sps_hit is (int32, int32, float)");
  sps::ScoreArgs x{};
  x.hits = reinterpret_cast<int3 *>(hits);
  x.hit_cap = capacity;
  x.hit_count = reinterpret_cast<unsigned long long *>(count);
  x.threshold = threshold;
  return score_one(q, items, chunk, sps::kModeThreshold, nullptr, nullptr, width, row_sums,
                   reinterpret_cast<hipStream_t>(stream), &x);
}

sps_status sps_items_half_workspace_size(const sps_items *h, size_t *bytes) {
  if (!h || !bytes) return fail(SPS_ERR_INVALID_ARGUMENT, "NULL argument");
  *bytes = (size_t)(h->nnz + sps::kPostPad4) * sizeof(uint32_t);
  return SPS_OK;
}

sps_status sps_items_enable_half(sps_items *h, void *workspace, size_t workspace_bytes,
                                 void *stream) {
  if (!h) return fail(SPS_ERR_INVALID_ARGUMENT, "NULL handle");
  size_t need = 0;
  sps_items_half_workspace_size(h, &need);
  if (!workspace || workspace_bytes < need)
    return fail(SPS_ERR_WORKSPACE_TOO_SMALL, "half workspace: %zu bytes needed", need);
  if (reinterpret_cast<uintptr_t>(workspace) & 15)
    return fail(SPS_ERR_INVALID_ARGUMENT, "half workspace must be 16-byte aligned");
  const hipError_t e = sps::launch_pack_half(h->post, h->nnz, static_cast<uint32_t *>(workspace),
                                             reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "sps_items_enable_half");
  h->post4 = static_cast<uint32_t *>(workspace);
  return SPS_OK;
}

sps_status sps_cosine_chunk_half(const sps_queries *q, const sps_items *items, int32_t chunk,
                                 uint16_t *out, int64_t ld_out, double *row_sums, void *stream) {
  sps_status st = check_score_args(q, items, out, ld_out);
  if (st != SPS_OK) return st;
  if (!items->post4)
    return fail(SPS_ERR_INVALID_ARGUMENT, "sps_items_enable_half has not been called");
  if (chunk < 0 || chunk >= items->g.num_chunks)
    return fail(SPS_ERR_CHUNK_RANGE, "chunk %d outside [0, %d)", chunk, items->g.num_chunks);
  return score_one(q, items, chunk, sps::kModeHalf, nullptr, out, ld_out, row_sums,
                   reinterpret_cast<hipStream_t>(stream));
}

sps_status sps_cosine_stream(const sps_queries *q, const sps_items *items, int32_t chunk_begin,
                             int32_t chunk_end, float *out, int64_t ld_out, double *row_sums,
                             void *stream) {
  sps_status st = check_score_args(q, items, out, ld_out);
  if (st != SPS_OK) return st;
  if (chunk_begin < 0 || chunk_end > items->g.num_chunks || chunk_begin > chunk_end)
    return fail(SPS_ERR_CHUNK_RANGE, "chunk range [%d, %d) outside [0, %d)", chunk_begin,
                chunk_end, items->g.num_chunks);
  for (int32_t c = chunk_begin; c < chunk_end; ++c) {
    double *rs = row_sums ? row_sums + (int64_t)(c - chunk_begin) * q->n_rows : nullptr;
    st = score_one(q, items, c, sps::kModeExact, out, nullptr, ld_out, rs,
                   reinterpret_cast<hipStream_t>(stream));
    if (st != SPS_OK) return st;
  }
  return SPS_OK;
}

sps_status sps_cosine_stream_host(const sps_queries *q, const sps_items *items,
                                  int32_t chunk_begin, int32_t chunk_end, float *host_out,
                                  int64_t ld_host, float *dev_buf0, float *dev_buf1,
                                  int64_t ld_dev, double *row_sums, void *stream,
                                  void *copy_stream) {
  sps_status st = check_score_args(q, items, dev_buf0, ld_dev);
  if (st != SPS_OK) return st;
  if (chunk_begin < 0 || chunk_end > items->g.num_chunks || chunk_begin > chunk_end)
    return fail(SPS_ERR_CHUNK_RANGE, "chunk range [%d, %d) outside [0, %d)", chunk_begin,
                chunk_end, items->g.num_chunks);
  if (chunk_begin == chunk_end || q->n_rows == 0) return SPS_OK;
  if (!dev_buf1 || dev_buf1 == dev_buf0)
    return fail(SPS_ERR_INVALID_ARGUMENT, "two distinct device buffers are needed");
  if (!host_out) return fail(SPS_ERR_INVALID_ARGUMENT, "NULL host output");
  const int64_t item0 = items->g.chunk_begin(chunk_begin);
  const int64_t span = items->g.chunk_end(chunk_end - 1) - item0;
  if (ld_host < span)
    return fail(SPS_ERR_INVALID_ARGUMENT, "ld_host %lld below the range's %lld items",
                (long long)ld_host, (long long)span);
  if ((uint64_t)ld_host > (uint64_t)INT64_MAX / 4 / (uint64_t)q->n_rows)
    return fail(SPS_ERR_OVERFLOW, "n_rows * ld_host overflows");
  // the copy engine overlaps only with page-locked host memory
  hipPointerAttribute_t attr;
  const hipError_t pe = hipPointerGetAttributes(&attr, host_out);
  if (pe != hipSuccess || attr.type != hipMemoryTypeHost) {
    (void)hipGetLastError();  // an unregistered pointer leaves an error behind
    return fail(SPS_ERR_INVALID_ARGUMENT,
                "host_out must be page-locked host memory (hipHostMalloc)");
  }
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const hipStream_t cs = reinterpret_cast<hipStream_t>(copy_stream);
  float *buf[2] = {dev_buf0, dev_buf1};
  hipEvent_t scored[2] = {nullptr, nullptr}, copied[2] = {nullptr, nullptr};
  bool recorded[2] = {false, false};  // copied[k] marks an enqueued copy
  bool unmarked = false;
  hipError_t e = hipSuccess;
  for (int k = 0; k < 2 && e == hipSuccess; ++k) {
    e = hipEventCreateWithFlags(&scored[k], hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&copied[k], hipEventDisableTiming);
  }
  for (int32_t c = chunk_begin; c < chunk_end && e == hipSuccess; ++c) {
    const int k = (c - chunk_begin) & 1;
    // buffer k is free once the copy of the chunk before last has left it
    if (c - chunk_begin >= 2) e = hipStreamWaitEvent(s, copied[k], 0);
    if (e != hipSuccess) break;
    double *rs = row_sums ? row_sums + (int64_t)(c - chunk_begin) * q->n_rows : nullptr;
    st = score_one(q, items, c, sps::kModeExact, buf[k], nullptr, ld_dev, rs, s);
    if (st != SPS_OK) break;
    e = hipEventRecord(scored[k], s);
    if (e == hipSuccess) e = hipStreamWaitEvent(cs, scored[k], 0);
    const int64_t len = items->g.chunk_end(c) - items->g.chunk_begin(c);
    if (e == hipSuccess)
      e = hipMemcpy2DAsync(host_out + (items->g.chunk_begin(c) - item0), (size_t)ld_host * 4,
                           buf[k], (size_t)ld_dev * 4, (size_t)len * 4, (size_t)q->n_rows,
                           hipMemcpyDeviceToHost, cs);
    if (e == hipSuccess) {
      e = hipEventRecord(copied[k], cs);
      if (e == hipSuccess) recorded[k] = true;
      else unmarked = true;  // a copy no event marks: wait for the copy stream below
    }
  }
  // the call completes in `stream` order: the stream waits for every copy
  // that was enqueued, also after an error, so that later work on `stream`
  // (the caller freeing or reusing the buffers) never overtakes a copy
  for (int k = 0; k < 2; ++k)
    if (recorded[k]) {
      const hipError_t w = hipStreamWaitEvent(s, copied[k], 0);
      if (e == hipSuccess) e = w;
    }
  if (unmarked) (void)hipStreamSynchronize(cs);
  for (int k = 0; k < 2; ++k) {
    if (scored[k]) (void)hipEventDestroy(scored[k]);
    if (copied[k]) (void)hipEventDestroy(copied[k]);
  }
  if (st != SPS_OK) return st;
  if (e != hipSuccess) return hip_fail(e, "sps_cosine_stream_host");
  return SPS_OK;
}

// ---- Block-Sparse CSR codec ----

// at most three varint bytes per entry of an int32 column: the byte
// positions stay below 2^31
constexpr int64_t kBscMaxNnz = kI32Max / 3;

static int64_t bsc_offsets_needed(int64_t nnz) { return (10 * nnz + 7) / 8; }

sps_status sps_bsc_offsets_bytes(int64_t nnz, size_t *bytes) {
  if (!bytes || nnz < 0) return fail(SPS_ERR_INVALID_ARGUMENT, "NULL argument or negative nnz");
  if (nnz > kBscMaxNnz)
    return fail(SPS_ERR_OVERFLOW, "nnz %lld above the codec's %lld", (long long)nnz,
                (long long)kBscMaxNnz);
  *bytes = (size_t)((bsc_offsets_needed(nnz) + 3) / 4 * 4);
  return SPS_OK;
}

sps_status sps_bsc_encode_sizes(const sps_csr *m, int32_t *bptr, void *scratch, void *stream,
                                int64_t *block_bytes) {
  if (block_bytes) *block_bytes = 0;
  sps_status st = check_csr_shape(m, "csr");
  if (st != SPS_OK) return st;
  if (!bptr || !block_bytes) return fail(SPS_ERR_INVALID_ARGUMENT, "NULL bptr or block_bytes");
  if (m->nnz > kBscMaxNnz)
    return fail(SPS_ERR_OVERFLOW, "nnz %lld above the codec's %lld", (long long)m->nnz,
                (long long)kBscMaxNnz);
  st = sps_validate_csr(m, scratch, stream, nullptr, nullptr);
  if (st != SPS_OK) return st;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = sps::launch_bsc_row_bytes(m->n_rows, m->nnz, m->indptr, m->indices, bptr, s);
  int32_t total = 0;
  if (e == hipSuccess)
    e = hipMemcpyAsync(&total, bptr + m->n_rows, sizeof total, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "sps_bsc_encode_sizes");
  *block_bytes = total;
  return SPS_OK;
}

sps_status sps_bsc_encode(const sps_csr *m, const int32_t *bptr, uint8_t *blocks,
                          int64_t block_bytes, uint8_t *offsets, int64_t offsets_bytes,
                          void *stream) {
  sps_status st = check_csr_shape(m, "csr");
  if (st != SPS_OK) return st;
  if (m->nnz > kBscMaxNnz) return fail(SPS_ERR_OVERFLOW, "nnz above the codec's limit");
  if (!bptr || block_bytes < 0 || (block_bytes > 0 && !blocks))
    return fail(SPS_ERR_INVALID_ARGUMENT, "NULL bptr or blocks, or negative block_bytes");
  size_t need = 0;
  sps_bsc_offsets_bytes(m->nnz, &need);
  if (offsets_bytes < (int64_t)need || (need > 0 && !offsets))
    return fail(SPS_ERR_WORKSPACE_TOO_SMALL, "offsets: %zu bytes needed", need);
  if (reinterpret_cast<uintptr_t>(offsets) & 3)
    return fail(SPS_ERR_INVALID_ARGUMENT, "offsets must be 4-byte aligned");
  const hipError_t e = sps::launch_bsc_encode(
      m->n_rows, m->nnz, m->indptr, m->indices, bptr, blocks, block_bytes,
      reinterpret_cast<uint32_t *>(offsets), (int64_t)need / 4,
      reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "sps_bsc_encode");
  return SPS_OK;
}

sps_status sps_bsc_decode(const sps_bsc *b, int32_t *indices, int32_t *status, void *stream) {
  if (!b) return fail(SPS_ERR_INVALID_ARGUMENT, "NULL matrix");
  if (b->n_rows < 0 || b->nnz < 0 || b->block_bytes < 0 || b->offsets_bytes < 0)
    return fail(SPS_ERR_INVALID_ARGUMENT, "negative size");
  if (b->n_rows >= kI32Max || b->nnz > kBscMaxNnz || b->block_bytes >= kI32Max)
    return fail(SPS_ERR_OVERFLOW, "sizes above the codec's limits");
  if (!b->indptr || !b->bptr || (b->block_bytes > 0 && !b->blocks))
    return fail(SPS_ERR_INVALID_ARGUMENT, "NULL indptr, bptr or blocks");
  if (b->nnz > 0 && (!indices || !b->offsets))
    return fail(SPS_ERR_INVALID_ARGUMENT, "NULL indices or offsets");
  if (b->offsets_bytes < bsc_offsets_needed(b->nnz))
    return fail(SPS_ERR_INVALID_ARGUMENT, "offsets: %lld bytes, %lld needed",
                (long long)b->offsets_bytes, (long long)bsc_offsets_needed(b->nnz));
  const hipError_t e = sps::launch_bsc_decode(b->n_rows, b->nnz, b->indptr, b->bptr,
                                              b->block_bytes, b->blocks, b->offsets, indices,
                                              status, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "sps_bsc_decode");
  return SPS_OK;
}

sps_status sps_row_inv_norms(const sps_csr *rows, float *inv_norm, void *stream) {
  sps_status st = check_csr_shape(rows, "rows");
  if (st != SPS_OK) return st;
  if (rows->n_rows > 0 && !inv_norm) return fail(SPS_ERR_INVALID_ARGUMENT, "NULL inv_norm");
  const hipError_t e = sps::launch_row_norms(rows->n_rows, rows->nnz, rows->indptr, rows->values,
                                             nullptr, inv_norm, nullptr,
                                             reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "sps_row_inv_norms");
  return SPS_OK;
}

sps_status sps_validate_csr(const sps_csr *m, void *scratch, void *stream,
                            int64_t *first_bad_row, int32_t *reason) {
  if (first_bad_row) *first_bad_row = -1;
  if (reason) *reason = 0;
  sps_status st = check_csr_shape(m, "csr");
  if (st != SPS_OK) return st;
  if (!scratch) return fail(SPS_ERR_INVALID_ARGUMENT, "NULL scratch");
  if (reinterpret_cast<uintptr_t>(scratch) & 7)
    return fail(SPS_ERR_INVALID_ARGUMENT, "scratch must be 8-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = sps::launch_csr_check(m->n_rows, m->n_cols, m->nnz, m->indptr, m->indices,
                                       m->values, 1, static_cast<int32_t *>(scratch), s);
  if (e != hipSuccess) return hip_fail(e, "sps_validate_csr");
  int32_t flags[4];
  e = hipMemcpyAsync(flags, scratch, sizeof flags, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "sps_validate_csr");
  if (flags[0] == 0 && flags[1] == 0) return SPS_OK;
  uint64_t key;
  memcpy(&key, flags + 2, sizeof key);
  if (first_bad_row) *first_bad_row = (int64_t)(key >> 3);
  if (reason) *reason = (int32_t)(key & 7);
  return fail(SPS_ERR_BAD_CSR, "non-canonical CSR at row %lld", (long long)(key >> 3));
}

}  // extern "C"
