"""Float64 CPU oracle for exact all-pairs sparse cosine similarity.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The GPU library
never imports, links or calls it, and this package imports nothing from the
GPU library.

Everything it computes is written out in ``sps_oracle.c`` (plain C, float64,
one pair at a time) after the page "稀疏嵌入批量相似度计算的工程化实践"
(Engineering practice of bulk similarity for sparse embeddings):

* ``row_norms``      -- §5.2 detail one: norm from the stored nonzeros only.
* ``chunk_csc``      -- §4.4 chunk slicing; a stable counting-sort transpose of
                        the chunk (the inverted lists the GPU builds).
* ``scores``         -- §3.1: cosine = dot / (|u| |v|), dot over the shared
                        support found by a two-pointer merge of the sorted index
                        arrays; §4.4: division by the norms after the dot.
* ``chunk_row_sums`` / ``col_sums`` -- closed forms by linearity of the dot
                        product, used to check chunks too big to merge pair by pair.

``oracle/bsc.py`` holds the Block-Sparse CSR codec of §3.2 (block ids
delta + variable-length coded, 10-bit packed local offsets) in plain Python
and numpy, pinned in tests/test_oracle_bsc.py.

Pins (tests/test_oracle_pins.py) tie every function to something other than
itself: brute-force dense dot products, scipy's sparse product, hand-worked
closed forms, invariants of the cosine, and transposition by scipy.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "sps_oracle.c")
DEFAULT_LIB = os.path.join(_HERE, "libsps_oracle.so")

_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def build(path: str = DEFAULT_LIB, mutant: int = 0, force: bool = False) -> str:
    """Compile the oracle with gcc. ``mutant`` > 0 plants a known mistake (tests only)."""
    if force or mutant or not os.path.exists(path) or \
            os.path.getmtime(path) < os.path.getmtime(SOURCE):
        tmp = path + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
               "-ffp-contract=off", "-DORC_MUTANT=%d" % mutant, "-o", tmp, SOURCE, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, path)
    return path


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _a(x, dtype):
    a = np.ascontiguousarray(x, dtype=dtype)
    return a


class Oracle:
    """ctypes front-end of one build of ``sps_oracle.c``."""

    def __init__(self, lib_path: str | None = None):
        self.path = lib_path or build()
        L = ctypes.CDLL(self.path)
        L.orc_validate_csr.restype = ctypes.c_int
        L.orc_validate_csr.argtypes = [_I64, _I64, _I64, _P, _P, _P, _P]
        L.orc_row_norms.restype = None
        L.orc_row_norms.argtypes = [_I64, _P, _P, _P, _P]
        L.orc_chunk_csc.restype = None
        L.orc_chunk_csc.argtypes = [_I64, _P, _P, _P, _P, _I64, _I64, _P, _P, _P]
        L.orc_scores.restype = None
        L.orc_scores.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _P,
                                 ctypes.c_int]
        L.orc_set_thread_cpus.restype = None
        L.orc_set_thread_cpus.argtypes = [_P, ctypes.c_int]
        L.orc_chunk_row_sums.restype = None
        L.orc_chunk_row_sums.argtypes = [_P, _P, _P, _P, _I64, _P, _P, _P, _P, _I64, _I64,
                                         _I64, _P, ctypes.c_int, ctypes.c_int]
        L.orc_col_sums.restype = None
        L.orc_col_sums.argtypes = [_P, _P, _P, _P, _I64, _P, _P, _P, _P, _I64, _I64, _I64, _P,
                                   ctypes.c_int]
        self.L = L

    # -- validation -------------------------------------------------------
    def validate(self, m) -> tuple[int, int]:
        ip = _a(m.indptr, np.int32)
        ix = _a(m.indices, np.int32)
        v = _a(m.values, np.float32)
        bad = _I64(-1)
        rc = self.L.orc_validate_csr(m.n_rows, m.n_cols, int(ip[-1]) if len(ip) else 0,
                                     ip.ctypes.data, ix.ctypes.data, v.ctypes.data,
                                     ctypes.byref(bad))
        return rc, bad.value

    # -- norms ------------------------------------------------------------
    def row_norms(self, m):
        """(norm64 float64[n], inv32 float32[n]) with inv32 = fl32(1/norm64), 0 if norm is 0."""
        ip = _a(m.indptr, np.int32)
        v = _a(m.values, np.float32)
        n64 = np.empty(m.n_rows, dtype=np.float64)
        inv = np.empty(m.n_rows, dtype=np.float32)
        self.L.orc_row_norms(m.n_rows, ip.ctypes.data, v.ctypes.data, n64.ctypes.data,
                             inv.ctypes.data)
        return n64, inv

    # -- inverted lists of one chunk --------------------------------------
    def chunk_csc(self, items, norm64, item_begin: int, item_end: int):
        """Reference CSC of items [item_begin, item_end): (col_ptr[dim+1], row[nnz_c], val[nnz_c])."""
        ip = _a(items.indptr, np.int32)
        ix = _a(items.indices, np.int32)
        v = _a(items.values, np.float32)
        n64 = _a(norm64, np.float64)
        cnnz = int(ip[item_end]) - int(ip[item_begin])
        col_ptr = np.empty(items.n_cols + 1, dtype=np.int32)
        row = np.empty(cnnz, dtype=np.int32)
        val = np.empty(cnnz, dtype=np.float32)
        self.L.orc_chunk_csc(items.n_cols, ip.ctypes.data, ix.ctypes.data, v.ctypes.data,
                             n64.ctypes.data, item_begin, item_end, col_ptr.ctypes.data,
                             row.ctypes.data, val.ctypes.data)
        return col_ptr, row, val

    # -- scores -----------------------------------------------------------
    def scores(self, queries, items, q_norm=None, i_norm=None, q_rows=None,
               item_begin: int = 0, item_end: int | None = None, n_threads: int | None = None,
               pin_cpus=None):
        """float64 S[q_rows x items[item_begin:item_end]] by per-pair merge.

        pin_cpus: optional CPU ids; thread t (the caller is thread 0) then runs on
        pin_cpus[t % len(pin_cpus)] (placement only, for timing)."""
        if q_norm is None:
            q_norm = self.row_norms(queries)[0]
        if i_norm is None:
            i_norm = self.row_norms(items)[0]
        if item_end is None:
            item_end = items.n_rows
        assert queries.n_cols == items.n_cols
        qip, qix, qv = _a(queries.indptr, np.int32), _a(queries.indices, np.int32), \
            _a(queries.values, np.float32)
        iip, iix, iv = _a(items.indptr, np.int32), _a(items.indices, np.int32), \
            _a(items.values, np.float32)
        qn, inn = _a(q_norm, np.float64), _a(i_norm, np.float64)
        if q_rows is None:
            rows_p = None
            n_sel = queries.n_rows
        else:
            rows = _a(q_rows, np.int64)
            rows_p = rows.ctypes.data
            n_sel = len(rows)
        out = np.empty((n_sel, item_end - item_begin), dtype=np.float64)
        cpus = None if not pin_cpus else _a(list(pin_cpus), np.int32)
        if cpus is not None:
            self.L.orc_set_thread_cpus(cpus.ctypes.data, len(cpus))
        try:
            self.L.orc_scores(qip.ctypes.data, qix.ctypes.data, qv.ctypes.data, qn.ctypes.data,
                              iip.ctypes.data, iix.ctypes.data, iv.ctypes.data, inn.ctypes.data,
                              rows_p, n_sel, item_begin, item_end, out.ctypes.data,
                              n_threads or _threads())
        finally:
            if cpus is not None:
                self.L.orc_set_thread_cpus(None, 0)
        return out

    # -- closed-form checksums -------------------------------------------
    def chunk_row_sums(self, queries, items, chunk_size: int, q_norm=None, i_norm=None,
                       n_threads: int | None = None, kind: int = 0):
        """float64 [n_chunks, n_q]: sum of S over each chunk's items, per query row.

        kind 1: the same sum of sum_d |q^_d i^_d| (the scale of each pair's rounding
        error); kind 2: of the number of shared stored dims (rows with a zero norm
        count none)."""
        if q_norm is None:
            q_norm = self.row_norms(queries)[0]
        if i_norm is None:
            i_norm = self.row_norms(items)[0]
        n_chunks = (items.n_rows + chunk_size - 1) // chunk_size
        out = np.empty((n_chunks, queries.n_rows), dtype=np.float64)
        qip, qix, qv = _a(queries.indptr, np.int32), _a(queries.indices, np.int32), \
            _a(queries.values, np.float32)
        iip, iix, iv = _a(items.indptr, np.int32), _a(items.indices, np.int32), \
            _a(items.values, np.float32)
        qn, inn = _a(q_norm, np.float64), _a(i_norm, np.float64)
        self.L.orc_chunk_row_sums(qip.ctypes.data, qix.ctypes.data, qv.ctypes.data,
                                  qn.ctypes.data, queries.n_rows, iip.ctypes.data,
                                  iix.ctypes.data, iv.ctypes.data, inn.ctypes.data,
                                  items.n_rows, items.n_cols, chunk_size, out.ctypes.data,
                                  n_threads or _threads(), int(kind))
        return out

    def col_sums(self, queries, items, item_begin: int = 0, item_end: int | None = None,
                 q_norm=None, i_norm=None, kind: int = 0):
        """float64 [item_end-item_begin]: sum over all query rows of S[q, i] (kind 1 and 2
        as in chunk_row_sums)."""
        if q_norm is None:
            q_norm = self.row_norms(queries)[0]
        if i_norm is None:
            i_norm = self.row_norms(items)[0]
        if item_end is None:
            item_end = items.n_rows
        out = np.empty(item_end - item_begin, dtype=np.float64)
        qip, qix, qv = _a(queries.indptr, np.int32), _a(queries.indices, np.int32), \
            _a(queries.values, np.float32)
        iip, iix, iv = _a(items.indptr, np.int32), _a(items.indices, np.int32), \
            _a(items.values, np.float32)
        qn, inn = _a(q_norm, np.float64), _a(i_norm, np.float64)
        self.L.orc_col_sums(qip.ctypes.data, qix.ctypes.data, qv.ctypes.data, qn.ctypes.data,
                            queries.n_rows, iip.ctypes.data, iix.ctypes.data, iv.ctypes.data,
                            inn.ctypes.data, items.n_cols, item_begin, item_end,
                            out.ctypes.data, int(kind))
        return out


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default
