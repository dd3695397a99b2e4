"""Exact all-pairs cosine similarity of sparse embeddings on MI355X (gfx950).

Thin Python binding of the C ABI in ``include/sps.h`` (``libsps.so``).
Arguments are marshalled here; every step of the computation runs in the
library's HIP kernels. PyTorch only provides device memory and streams.

Page followed: "稀疏嵌入批量相似度计算的工程化实践" (Engineering practice of
bulk similarity for sparse embeddings): §3.1 defines the cosine over the
shared support, §5.2 the norms, §2.2 and §4.4 the item-chunk streaming with
8192-item chunks, §2.3 the full float32 output.

Typical use::

    items = sps.prepare(sps.CSR.from_host(item_csr, "cuda"), chunk_size=8192)
    queries = sps.prepare_queries(sps.CSR.from_host(query_csr, "cuda"), items)
    out = torch.empty(n_query, 8192, device="cuda")
    for c in range(items.num_chunks):
        sps.cosine_chunk(queries, items, c, out)   # out[:, :chunk_len] = S[:, chunk c]
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsps.so")

SPS_OK = 0
_STATUS = {
    0: "SPS_OK", -1: "SPS_ERR_INVALID_ARGUMENT", -2: "SPS_ERR_BAD_CSR",
    -3: "SPS_ERR_DIM_MISMATCH", -4: "SPS_ERR_WORKSPACE_TOO_SMALL", -5: "SPS_ERR_CHUNK_RANGE",
    -6: "SPS_ERR_OVERFLOW", -7: "SPS_ERR_HIP", -8: "SPS_ERR_UNSUPPORTED",
}


class SpsError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s: %s" % (_STATUS.get(status, status), msg))
        self.status = status


class _Csr(ctypes.Structure):
    _fields_ = [("n_rows", ctypes.c_int64), ("n_cols", ctypes.c_int64), ("nnz", ctypes.c_int64),
                ("indptr", ctypes.c_void_p), ("indices", ctypes.c_void_p),
                ("values", ctypes.c_void_p)]


class _Bsc(ctypes.Structure):
    _fields_ = [("n_rows", ctypes.c_int64), ("n_cols", ctypes.c_int64), ("nnz", ctypes.c_int64),
                ("indptr", ctypes.c_void_p), ("bptr", ctypes.c_void_p),
                ("blocks", ctypes.c_void_p), ("block_bytes", ctypes.c_int64),
                ("offsets", ctypes.c_void_p), ("offsets_bytes", ctypes.c_int64),
                ("values", ctypes.c_void_p)]


class _SliceView(ctypes.Structure):
    _fields_ = [("item_begin", ctypes.c_int64), ("slice_len", ctypes.c_int32),
                ("slice_nnz", ctypes.c_int32), ("post", ctypes.c_void_p),
                ("item_inv_norm", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t

# name -> (restype, argtypes); every symbol include/sps.h declares
SIGNATURES = {
    "sps_items_workspace_size": (_I32, [_I64, _I64, _I64, _I32, ctypes.POINTER(_SZ),
                                        ctypes.POINTER(_SZ)]),
    "sps_prepare": (_I32, [ctypes.POINTER(_Csr), _I32, _P, _SZ, _P, _SZ, _P,
                           ctypes.POINTER(_P)]),
    "sps_items_info": (_I32, [_P, ctypes.POINTER(_I64), ctypes.POINTER(_I64),
                              ctypes.POINTER(_I64), ctypes.POINTER(_I32), ctypes.POINTER(_I32)]),
    "sps_items_slices": (_I32, [_P, ctypes.POINTER(_I32), ctypes.POINTER(_I32),
                                ctypes.POINTER(_I64)]),
    "sps_items_slice_view": (_I32, [_P, _I64, _P, ctypes.POINTER(_SliceView)]),
    "sps_items_slice_col_ptr": (_I32, [_P, _I64, _P, _P, _P]),
    "sps_items_heavy_dims": (_I32, [_P, _P, _P, _I32, ctypes.POINTER(_I32)]),
    "sps_items_destroy": (None, [_P]),
    "sps_queries_workspace_size": (_I32, [_P, _I64, _I64, _I64, ctypes.POINTER(_SZ)]),
    "sps_prepare_queries": (_I32, [ctypes.POINTER(_Csr), _P, _P, _SZ, _P, ctypes.POINTER(_P)]),
    "sps_queries_inv_norms": (_I32, [_P, ctypes.POINTER(_P)]),
    "sps_queries_destroy": (None, [_P]),
    "sps_cosine_chunk": (_I32, [_P, _P, _I32, _P, _I64, _P, _P]),
    "sps_cosine_chunk_static": (_I32, [_P, _P, _I32, _P, _I64, _P, _P]),
    "sps_cosine_stream": (_I32, [_P, _P, _I32, _I32, _P, _I64, _P, _P]),
    "sps_cosine_stream_host": (_I32, [_P, _P, _I32, _I32, _P, _I64, _P, _P, _I64, _P, _P, _P]),
    "sps_cosine_chunk_threshold": (_I32, [_P, _P, _I32, ctypes.c_float, _P, _I64, _P, _P, _P]),
    "sps_items_half_workspace_size": (_I32, [_P, ctypes.POINTER(_SZ)]),
    "sps_items_enable_half": (_I32, [_P, _P, _SZ, _P]),
    "sps_cosine_chunk_half": (_I32, [_P, _P, _I32, _P, _I64, _P, _P]),
    "sps_row_inv_norms": (_I32, [ctypes.POINTER(_Csr), _P, _P]),
    "sps_bsc_offsets_bytes": (_I32, [_I64, ctypes.POINTER(_SZ)]),
    "sps_bsc_encode_sizes": (_I32, [ctypes.POINTER(_Csr), _P, _P, _P, ctypes.POINTER(_I64)]),
    "sps_bsc_encode": (_I32, [ctypes.POINTER(_Csr), _P, _P, _I64, _P, _I64, _P]),
    "sps_bsc_decode": (_I32, [ctypes.POINTER(_Bsc), _P, _P, _P]),
    "sps_validate_csr": (_I32, [ctypes.POINTER(_Csr), _P, _P, ctypes.POINTER(_I64),
                                ctypes.POINTER(_I32)]),
    "sps_status_string": (ctypes.c_char_p, [_I32]),
    "sps_last_error_message": (ctypes.c_char_p, []),
}

_lib = None


def load_library(path: str | None = None):
    """Load libsps.so (building it with hipcc first if it is absent).

    There is no fallback: without the HIP library nothing here runs.
    """
    global _lib
    if _lib is not None and path is None:
        return _lib
    # torch ships its own HIP runtime and this library links the system one: the
    # process holds both, and torch's must initialise the GPU first
    if torch.cuda.is_available():
        torch.cuda.init()
    p = path or LIB_PATH
    if not os.path.exists(p):
        from . import _build
        _build.build()
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _check(st: int):
    if st != SPS_OK:
        msg = _lib.sps_last_error_message().decode(errors="replace")
        raise SpsError(st, msg)


def _stream_ptr(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _workspace(nbytes: int, device) -> tuple[torch.Tensor, int]:
    """uint8 device buffer of at least nbytes, 256-byte aligned."""
    buf = torch.empty(max(int(nbytes), 1) + 256, dtype=torch.uint8, device=device)
    p = buf.data_ptr()
    return buf, (p + 255) & ~255


# ---------------------------------------------------------------------------

@dataclass
class CSR:
    """Device CSR (int32 indptr/indices, float32 values) in torch tensors."""
    indptr: torch.Tensor
    indices: torch.Tensor
    values: torch.Tensor
    n_rows: int
    n_cols: int

    @property
    def nnz(self) -> int:
        return int(self.indices.numel())

    @classmethod
    def from_host(cls, m, device="cuda") -> "CSR":
        """From any object with numpy indptr/indices/values, n_rows, n_cols."""
        ip = torch.as_tensor(m.indptr).to(device=device, dtype=torch.int32).contiguous()
        ix = torch.as_tensor(m.indices).to(device=device, dtype=torch.int32).contiguous()
        v = torch.as_tensor(m.values).to(device=device, dtype=torch.float32).contiguous()
        return cls(ip, ix, v, int(m.n_rows), int(m.n_cols))

    def _c(self) -> _Csr:
        assert self.indptr.is_cuda and self.indices.is_cuda and self.values.is_cuda
        assert self.indptr.dtype == torch.int32 and self.indices.dtype == torch.int32
        assert self.values.dtype == torch.float32
        assert self.indptr.is_contiguous() and self.indices.is_contiguous() \
            and self.values.is_contiguous()
        assert self.indptr.numel() == self.n_rows + 1
        assert self.values.numel() == self.indices.numel()
        return _Csr(self.n_rows, self.n_cols, self.nnz, self.indptr.data_ptr(),
                    self.indices.data_ptr() if self.nnz else None,
                    self.values.data_ptr() if self.nnz else None)


@dataclass
class BSC:
    """Device Block-Sparse CSR (§3.2): the CSR's indptr and values, the per-row
    block-id varint bytes (located by bptr) and the packed 10-bit offsets."""
    indptr: torch.Tensor   # int32 [n_rows + 1]
    bptr: torch.Tensor     # int32 [n_rows + 1]
    blocks: torch.Tensor   # uint8 [bptr[-1]]
    offsets: torch.Tensor  # uint8, a multiple of 4 bytes
    values: torch.Tensor   # float32 [nnz]
    n_rows: int
    n_cols: int

    @property
    def nnz(self) -> int:
        return int(self.values.numel())

    def index_bytes(self) -> int:
        """Bytes that locate the entries: bptr, varints and offsets (indptr, as in
        the CSR, left out)."""
        return 4 * self.bptr.numel() + self.blocks.numel() + (10 * self.nnz + 7) // 8

    def _c(self) -> _Bsc:
        for t, dt in ((self.indptr, torch.int32), (self.bptr, torch.int32),
                      (self.blocks, torch.uint8), (self.offsets, torch.uint8),
                      (self.values, torch.float32)):
            assert t.is_cuda and t.dtype == dt and t.is_contiguous()
        return _Bsc(self.n_rows, self.n_cols, self.nnz, self.indptr.data_ptr(),
                    self.bptr.data_ptr(), self.blocks.data_ptr() if self.blocks.numel() else None,
                    self.blocks.numel(), self.offsets.data_ptr() if self.offsets.numel() else None,
                    self.offsets.numel(), self.values.data_ptr() if self.nnz else None)


def bsc_encode(m: CSR, stream=None) -> BSC:
    """Block-Sparse CSR of a canonical CSR (synchronises once, to size the varint
    stream; raises SpsError for a non-canonical CSR)."""
    load_library()
    dev = m.indptr.device
    c = m._c()
    bptr = torch.empty(m.n_rows + 1, dtype=torch.int32, device=dev)
    scratch = torch.empty(16, dtype=torch.int32, device=dev)
    nbytes = _I64()
    _check(_lib.sps_bsc_encode_sizes(ctypes.byref(c), bptr.data_ptr(), scratch.data_ptr(),
                                     _stream_ptr(stream), ctypes.byref(nbytes)))
    ob = _SZ()
    _check(_lib.sps_bsc_offsets_bytes(m.nnz, ctypes.byref(ob)))
    blocks = torch.empty(nbytes.value, dtype=torch.uint8, device=dev)
    offsets = torch.empty(ob.value, dtype=torch.uint8, device=dev)
    _check(_lib.sps_bsc_encode(ctypes.byref(c), bptr.data_ptr(),
                               blocks.data_ptr() if nbytes.value else None, nbytes.value,
                               offsets.data_ptr() if ob.value else None, ob.value,
                               _stream_ptr(stream)))
    return BSC(m.indptr, bptr, blocks, offsets, m.values, m.n_rows, m.n_cols)


def bsc_decode(b: BSC, stream=None, check: bool = True) -> CSR:
    """The CSR of a Block-Sparse CSR (its indptr and values shared). With check,
    synchronises and raises SpsError for a malformed encoding."""
    load_library()
    dev = b.indptr.device
    indices = torch.empty(b.nnz, dtype=torch.int32, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    c = b._c()
    _check(_lib.sps_bsc_decode(ctypes.byref(c), indices.data_ptr() if b.nnz else None,
                               status.data_ptr(), _stream_ptr(stream)))
    if check and int(status.item()) != 0:
        raise SpsError(-2, "malformed Block-Sparse CSR (status %d)" % int(status.item()))
    return CSR(b.indptr, indices, b.values, b.n_rows, b.n_cols)


class Items:
    """Prepared item corpus (owns its workspaces)."""

    def __init__(self, handle, persistent, scratch, src: CSR, chunk_size: int):
        self._h = handle
        self._persistent = persistent
        self._scratch = scratch
        self._src = src  # kept alive until release_inputs()
        n, d, z = _I64(), _I64(), _I64()
        cs, nc = _I32(), _I32()
        _check(_lib.sps_items_info(handle, ctypes.byref(n), ctypes.byref(d), ctypes.byref(z),
                                   ctypes.byref(cs), ctypes.byref(nc)))
        self.n_items, self.dim, self.nnz = n.value, d.value, z.value
        self.chunk_size, self.num_chunks = cs.value, nc.value
        ss, spc, ns = _I32(), _I32(), _I64()
        _check(_lib.sps_items_slices(handle, ctypes.byref(ss), ctypes.byref(spc), ctypes.byref(ns)))
        self.slice_size, self.slices_per_chunk, self.num_slices = ss.value, spc.value, ns.value

    def chunk_len(self, c: int) -> int:
        b = c * self.chunk_size
        return min(b + self.chunk_size, self.n_items) - b

    def enable_half(self, stream=None) -> None:
        """Build the fp16 postings used by cosine_chunk_half (once; needs the prepare work
        to have been enqueued on the same stream)."""
        if getattr(self, "_half", None) is not None:
            return
        n = _SZ()
        _check(_lib.sps_items_half_workspace_size(self._h, ctypes.byref(n)))
        buf, ptr = _workspace(n.value, self._persistent.device)
        _check(_lib.sps_items_enable_half(self._h, ptr, n.value, _stream_ptr(stream)))
        self._half = buf

    def release_inputs(self):
        """Drop the item CSR and prepare scratch (after the prepare work completed)."""
        torch.cuda.current_stream().synchronize()
        self._src = None
        self._scratch = None

    def slice_view(self, s: int, stream=None) -> dict:
        """Device views of slice s's inverted lists (synchronous)."""
        v = _SliceView()
        _check(_lib.sps_items_slice_view(self._h, s, _stream_ptr(stream), ctypes.byref(v)))
        dev = self._persistent.device

        def view(ptr, n, dtype, elem):
            if n == 0:
                return torch.empty(0, dtype=dtype, device=dev)
            base = self._persistent.data_ptr()
            off = ptr - base
            assert 0 <= off and off + n * elem <= self._persistent.numel()
            return self._persistent[off:off + n * elem].view(dtype)

        return {
            "item_begin": v.item_begin, "slice_len": v.slice_len, "slice_nnz": v.slice_nnz,
            # sps_posting records: int32 pairs (item id, value bits)
            "post": view(v.post, v.slice_nnz, torch.int32, 8).view(-1, 2),
            "item_inv_norm": view(v.item_inv_norm, v.slice_len, torch.float32, 4),
        }

    def slice_col_ptr(self, s: int, stream=None):
        """(col_ptr int32[dim+1], consistent: bool) of slice s, expanded from its dim index
        on the device (synchronous)."""
        dev = self._persistent.device
        cp = torch.empty(self.dim + 1, dtype=torch.int32, device=dev)
        st = torch.zeros(1, dtype=torch.int32, device=dev)
        _check(_lib.sps_items_slice_col_ptr(self._h, s, cp.data_ptr(), st.data_ptr(),
                                            _stream_ptr(stream)))
        (stream or torch.cuda.current_stream()).synchronize()
        return cp, int(st.item()) == 0

    def heavy_dims(self, stream=None) -> list:
        """The dims kept as dense rows (ascending; synchronous)."""
        buf = (_I32 * 128)()
        n = _I32()
        _check(_lib.sps_items_heavy_dims(self._h, _stream_ptr(stream), buf, 128, ctypes.byref(n)))
        return [int(buf[i]) for i in range(n.value)]

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h and _lib is not None:
            _lib.sps_items_destroy(h)


class Queries:
    """Prepared query batch (owns its workspace)."""

    def __init__(self, handle, ws, n_rows: int, items: Items):
        self._h = handle
        self._ws = ws
        self.n_rows = n_rows
        self.items = items
        p = _P()
        _check(_lib.sps_queries_inv_norms(handle, ctypes.byref(p)))
        off = p.value - ws.data_ptr()
        self.inv_norm = ws[off:off + 4 * n_rows].view(torch.float32) if n_rows else \
            torch.empty(0, dtype=torch.float32, device=ws.device)

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h and _lib is not None:
            _lib.sps_queries_destroy(h)


def items_workspace_size(n_items: int, dim: int, nnz: int, chunk_size: int) -> tuple[int, int]:
    load_library()
    p, s = _SZ(), _SZ()
    _check(_lib.sps_items_workspace_size(n_items, dim, nnz, chunk_size, ctypes.byref(p),
                                         ctypes.byref(s)))
    return p.value, s.value


def prepare(items, chunk_size: int = 8192, stream=None) -> Items:
    """Norms + per-chunk inverted lists of an item corpus (asynchronous). items is a
    CSR, or a BSC whose indices are decoded on the device first."""
    load_library()
    if isinstance(items, BSC):
        items = bsc_decode(items, stream)
    pb, sb = items_workspace_size(items.n_rows, items.n_cols, items.nnz, chunk_size)
    dev = items.indptr.device
    pbuf, pptr = _workspace(pb, dev)
    sbuf, sptr = _workspace(sb, dev)
    h = _P()
    c = items._c()
    _check(_lib.sps_prepare(ctypes.byref(c), chunk_size, pptr, pb, sptr, sb, _stream_ptr(stream),
                            ctypes.byref(h)))
    # the persistent view handed out by chunk_view is relative to the aligned base
    pview = pbuf[pptr - pbuf.data_ptr():]
    return Items(h.value, pview, sbuf, items, chunk_size)


def prepare_queries(queries: CSR, items: Items, stream=None) -> Queries:
    """Inverse norms and per-workgroup merged dim lists of a query batch (asynchronous)."""
    load_library()
    nb = _SZ()
    _check(_lib.sps_queries_workspace_size(items._h, queries.n_rows, queries.n_cols,
                                           queries.nnz, ctypes.byref(nb)))
    buf, ptr = _workspace(nb.value, queries.indptr.device)
    h = _P()
    c = queries._c()
    _check(_lib.sps_prepare_queries(ctypes.byref(c), items._h, ptr, nb.value, _stream_ptr(stream),
                                    ctypes.byref(h)))
    q = Queries(h.value, buf[ptr - buf.data_ptr():], queries.n_rows, items)
    q._src = queries
    return q


def _out_args(q: Queries, out: torch.Tensor, row_sums, dtype=torch.float32):
    assert out.is_cuda and out.dtype == dtype and out.dim() == 2
    assert out.stride(1) == 1 and out.shape[0] == q.n_rows
    ld = out.stride(0) if q.n_rows > 1 else out.shape[1]
    rs = None
    if row_sums is not None:
        assert row_sums.is_cuda and row_sums.dtype == torch.float64 and row_sums.is_contiguous()
        rs = row_sums.data_ptr()
    return ld, rs


def cosine_chunk(q: Queries, items: Items, chunk: int, out: torch.Tensor,
                 row_sums: torch.Tensor | None = None, stream=None) -> None:
    """out[:, :chunk_len] = S[:, chunk]; out is (n_query, >= chunk_len) float32, row-major."""
    ld, rs = _out_args(q, out, row_sums)
    assert out.shape[1] >= items.chunk_len(chunk)
    if row_sums is not None:
        assert row_sums.numel() >= q.n_rows
    _check(_lib.sps_cosine_chunk(q._h, items._h, chunk, out.data_ptr(), ld, rs,
                                 _stream_ptr(stream)))


def cosine_chunk_static(q: Queries, items: Items, chunk: int, out: torch.Tensor,
                        row_sums: torch.Tensor | None = None, stream=None) -> None:
    """cosine_chunk with the partial row sums in the library's static device scratch
    (no allocation; calls overlapping on one GPU race)."""
    ld, rs = _out_args(q, out, row_sums)
    assert out.shape[1] >= items.chunk_len(chunk)
    if row_sums is not None:
        assert row_sums.numel() >= q.n_rows
    _check(_lib.sps_cosine_chunk_static(q._h, items._h, chunk, out.data_ptr(), ld, rs,
                                        _stream_ptr(stream)))


def cosine_chunk_half(q: Queries, items: Items, chunk: int, out: torch.Tensor,
                      row_sums: torch.Tensor | None = None, stream=None) -> None:
    """The reduced-precision variant: out[:, :chunk_len] = fp16 scores from fp16 item
    values (|error| < 1e-3); out is (n_query, >= chunk_len) float16, row-major. Needs
    items.enable_half()."""
    ld, rs = _out_args(q, out, row_sums, torch.float16)
    assert out.shape[1] >= items.chunk_len(chunk)
    if row_sums is not None:
        assert row_sums.numel() >= q.n_rows
    _check(_lib.sps_cosine_chunk_half(q._h, items._h, chunk, out.data_ptr(), ld, rs,
                                      _stream_ptr(stream)))


def cosine_chunk_threshold(q: Queries, items: Items, chunk: int, threshold: float,
                           hits: torch.Tensor, count: torch.Tensor,
                           row_sums: torch.Tensor | None = None, stream=None) -> None:
    """Append every score >= threshold of the chunk to hits as (row, item, score bits) int32
    triples; count (one int64/uint64 device value, zeroed once by the caller) advances by the
    number of hits, including those past hits' capacity, which are dropped."""
    assert hits.is_cuda and hits.dtype == torch.int32 and hits.dim() == 2
    assert hits.shape[1] == 3 and hits.is_contiguous()
    assert count.is_cuda and count.dtype == torch.int64 and count.numel() >= 1
    rs = None
    if row_sums is not None:
        assert row_sums.is_cuda and row_sums.dtype == torch.float64 and row_sums.is_contiguous()
        assert row_sums.numel() >= q.n_rows
        rs = row_sums.data_ptr()
    _check(_lib.sps_cosine_chunk_threshold(q._h, items._h, chunk, float(threshold),
                                           hits.data_ptr() if hits.numel() else None,
                                           hits.shape[0], count.data_ptr(), rs,
                                           _stream_ptr(stream)))


def hits_to_numpy(hits: torch.Tensor, count: int):
    """(rows, items, scores) numpy arrays of the first min(count, capacity) hits."""
    h = hits[:min(int(count), hits.shape[0])].cpu().numpy()
    return h[:, 0].copy(), h[:, 1].copy(), h[:, 2].copy().view(np.float32)


def cosine_stream(q: Queries, items: Items, chunk_begin: int, chunk_end: int,
                  out: torch.Tensor, row_sums: torch.Tensor | None = None, stream=None) -> None:
    """Chunks [chunk_begin, chunk_end) in turn into the same rotating buffer `out`."""
    ld, rs = _out_args(q, out, row_sums)
    assert out.shape[1] >= min(items.chunk_size, items.n_items)
    if row_sums is not None:
        assert row_sums.numel() >= (chunk_end - chunk_begin) * q.n_rows
    _check(_lib.sps_cosine_stream(q._h, items._h, chunk_begin, chunk_end, out.data_ptr(), ld, rs,
                                  _stream_ptr(stream)))


_copy_streams: dict = {}


def _copy_stream(device) -> "torch.cuda.Stream":
    """One side stream per device for device-to-host copies (default priority)."""
    idx = torch.device(device).index
    idx = torch.cuda.current_device() if idx is None else idx
    if idx not in _copy_streams:
        _copy_streams[idx] = torch.cuda.Stream(device=idx)
    return _copy_streams[idx]


def cosine_stream_host(q: Queries, items: Items, chunk_begin: int, chunk_end: int,
                       host_out: torch.Tensor, bufs=None, row_sums: torch.Tensor | None = None,
                       stream=None, copy_stream=None) -> None:
    """Chunks [chunk_begin, chunk_end) into the pinned host matrix host_out
    (n_query x >= the range's items, float32, row-major), column 0 being item
    chunk_begin * chunk_size: scored into two alternating device buffers, each
    copied out by the copy engine on a side stream while the next is scored.
    Asynchronous in `stream` order: synchronise before reading host_out."""
    assert not host_out.is_cuda and host_out.is_pinned(), "host_out must be a pinned CPU tensor"
    assert host_out.dtype == torch.float32 and host_out.dim() == 2
    assert host_out.stride(1) == 1 and host_out.shape[0] == q.n_rows
    ld_host = host_out.stride(0) if q.n_rows > 1 else host_out.shape[1]
    if chunk_end > chunk_begin:
        span = min(chunk_end * items.chunk_size, items.n_items) - chunk_begin * items.chunk_size
        assert host_out.shape[1] >= span, "host_out narrower than the chunk range"
    s = stream if stream is not None else torch.cuda.current_stream()
    dev = s.device
    if bufs is None:
        width = max(min(items.chunk_size, items.n_items), 1)
        bufs = tuple(torch.empty(q.n_rows, width, dtype=torch.float32, device=dev)
                     for _ in range(2))
        for b in bufs:  # freed by the caller's stream order only after the copies
            b.record_stream(s)
    b0, b1 = bufs
    assert b0.is_cuda and b0.dtype == torch.float32 and b0.stride(1) == 1
    assert b1.shape == b0.shape and b1.stride() == b0.stride() and b1.dtype == b0.dtype
    assert b0.shape[0] == q.n_rows and b0.shape[1] >= min(items.chunk_size, items.n_items)
    ld_dev = b0.stride(0) if q.n_rows > 1 else b0.shape[1]
    rs = None
    if row_sums is not None:
        assert row_sums.is_cuda and row_sums.dtype == torch.float64 and row_sums.is_contiguous()
        assert row_sums.numel() >= (chunk_end - chunk_begin) * q.n_rows
        rs = row_sums.data_ptr()
    cs = copy_stream if copy_stream is not None else _copy_stream(dev)
    _check(_lib.sps_cosine_stream_host(q._h, items._h, chunk_begin, chunk_end,
                                       host_out.data_ptr(), ld_host, b0.data_ptr(),
                                       b1.data_ptr(), ld_dev, rs, int(s.cuda_stream),
                                       int(cs.cuda_stream)))


def row_inv_norms(m: CSR, stream=None) -> torch.Tensor:
    load_library()
    out = torch.empty(m.n_rows, dtype=torch.float32, device=m.indptr.device)
    c = m._c()
    _check(_lib.sps_row_inv_norms(ctypes.byref(c), out.data_ptr() if m.n_rows else None,
                                  _stream_ptr(stream)))
    return out


def validate_csr(m: CSR, stream=None) -> tuple[bool, int, int]:
    """(ok, first_bad_row, reason); reason 1 indptr, 2 order/dup, 3 range, 4 non-finite."""
    load_library()
    scratch = torch.empty(64, dtype=torch.uint8, device=m.indptr.device)
    row, why = _I64(), _I32()
    c = m._c()
    st = _lib.sps_validate_csr(ctypes.byref(c), scratch.data_ptr(), _stream_ptr(stream),
                               ctypes.byref(row), ctypes.byref(why))
    if st == -2:
        return False, row.value, why.value
    _check(st)
    return True, -1, 0


def bulk_similarity(queries: CSR, items: CSR, chunk_size: int = 8192, out=None,
                    on_chunk=None, row_sums: bool = False):
    """Full (n_query, n_item) float32 cosine matrix, item chunk by item chunk.

    Mirrors the streaming loop of §4.4 with every step on the GPU. With
    ``out`` (a device or pinned host tensor of shape (n_query, n_item)) each
    chunk is copied there; with ``on_chunk(c, buf, sums)`` each chunk's
    device buffer is handed to the callback instead (and reused after it
    returns). Returns ``out`` (allocated on the device if neither is given).
    """
    it = prepare(items, chunk_size)
    q = prepare_queries(queries, it)
    dev = queries.indptr.device
    if out is not None and on_chunk is None and not out.is_cuda and out.is_pinned():
        # pinned host output: double-buffered, the copies overlapping the scoring
        cosine_stream_host(q, it, 0, it.num_chunks, out)
        torch.cuda.current_stream().synchronize()
        return out
    width = min(chunk_size, it.n_items)
    buf = torch.empty(queries.n_rows, max(width, 1), dtype=torch.float32, device=dev)
    sums = torch.empty(queries.n_rows, dtype=torch.float64, device=dev) if row_sums else None
    if out is None and on_chunk is None:
        out = torch.empty(queries.n_rows, it.n_items, dtype=torch.float32, device=dev)
    for c in range(it.num_chunks):
        cosine_chunk(q, it, c, buf, sums)
        n = it.chunk_len(c)
        b = c * chunk_size
        if on_chunk is not None:
            on_chunk(c, buf[:, :n], sums)
        if out is not None:
            out[:, b:b + n].copy_(buf[:, :n], non_blocking=False)
    return out
