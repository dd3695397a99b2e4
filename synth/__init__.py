"""Seeded synthetic CSR corpora for the exact sparse-cosine path.

This package makes inputs only; it contains none of the similarity
arithmetic. The float64 oracle (``oracle``) and the GPU library
(``sparse_embedding_exact_amd``) are both fed from it, and neither is
imported here.

Workload shapes come from the page "稀疏嵌入批量相似度计算的工程化实践"
(Engineering practice of bulk similarity for sparse embeddings): §1 gives
the production shape (50,000 queries x 2,000,000 items, dim 1.2M, mean
nnz 43, BM25+TF-IDF title embeddings, not published), §2.2 and §4.4 give
the 8192-item chunk. The private data is replaced by seeded draws:
positive heavy-tailed weights become lognormal(0, 1) and the term-id skew
(§3.2: ids cluster in a dictionary prefix) becomes a bounded Zipf law whose
heaviest ranks are the lowest dims.

Random numbers come from Philox4x32-10 (Salmon et al., SC'11), one counter
stream per (matrix, row, purpose), implemented in ``synth.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")


def build(force: bool = False) -> str:
    """Compile ``synth.c`` into ``libsynth.so`` (host code, gcc)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Spec(ctypes.Structure):
    _fields_ = [
        ("n_rows", ctypes.c_int64), ("dim", ctypes.c_int64), ("seed", ctypes.c_uint64),
        ("matrix", ctypes.c_uint32), ("nnz_kind", ctypes.c_int),
        ("nnz_a", ctypes.c_double), ("nnz_b", ctypes.c_double),
        ("nnz_min", ctypes.c_int64), ("nnz_max", ctypes.c_int64),
        ("idx_kind", ctypes.c_int), ("zipf_s", ctypes.c_double), ("val_kind", ctypes.c_int),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        lib.synth_row_nnz.restype = ctypes.c_int64
        lib.synth_row_nnz.argtypes = [ctypes.POINTER(_Spec), ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_int]
        lib.synth_fill.restype = ctypes.c_int
        lib.synth_fill.argtypes = [ctypes.POINTER(_Spec), ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_int]
        lib.synth_subset.restype = ctypes.c_int
        lib.synth_subset.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64,
                                     ctypes.c_int64, ctypes.c_void_p]
        lib.synth_philox4x32_10.restype = None
        lib.synth_philox4x32_10.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        _lib = lib
    return _lib


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


@dataclass
class HostCSR:
    """Canonical CSR on the host: int32 indptr/indices, float32 values."""
    indptr: np.ndarray
    indices: np.ndarray
    values: np.ndarray
    n_rows: int
    n_cols: int

    @property
    def nnz(self) -> int:
        return int(self.indptr[-1])

    def row(self, r: int):
        b, e = int(self.indptr[r]), int(self.indptr[r + 1])
        return self.indices[b:e], self.values[b:e]

    def take_rows(self, rows) -> "HostCSR":
        rows = np.asarray(rows, dtype=np.int64)
        lens = (self.indptr[rows + 1] - self.indptr[rows]).astype(np.int64)
        indptr = np.zeros(len(rows) + 1, dtype=np.int64)
        np.cumsum(lens, out=indptr[1:])
        total = int(indptr[-1])
        starts = self.indptr[rows].astype(np.int64)
        # gather positions of every entry of the selected rows, in order
        pos = np.repeat(starts - indptr[:-1], lens) + np.arange(total, dtype=np.int64)
        return HostCSR(indptr.astype(np.int32), self.indices[pos].copy(),
                       self.values[pos].copy(), len(rows), self.n_cols)

    def to_scipy(self):
        import scipy.sparse as sp
        return sp.csr_matrix((self.values, self.indices, self.indptr),
                             shape=(self.n_rows, self.n_cols))


NNZ_UNIFORM, NNZ_POISSON, NNZ_LOGNORMAL = 0, 1, 2
IDX_UNIFORM, IDX_ZIPF = 0, 1
VAL_LOGNORMAL, VAL_LOG1P_HALFNORMAL, VAL_NORMAL = 0, 1, 2


def make_corpus(n_rows: int, dim: int, seed: int, matrix: int, *, nnz: tuple, idx: tuple,
                val: int, force_empty: np.ndarray | None = None,
                n_threads: int | None = None) -> HostCSR:
    """Draw one CSR corpus.

    nnz: ("uniform", lo, hi) | ("poisson", lam, min) | ("lognormal", mu, sigma, lo, hi)
    idx: ("uniform",) | ("zipf", s)   -- rows hold distinct dims, ascending
    val: VAL_* code
    """
    lib = _load()
    s = _Spec()
    s.n_rows, s.dim, s.seed, s.matrix = n_rows, dim, seed, matrix
    s.nnz_min, s.nnz_max = 0, dim
    if nnz[0] == "uniform":
        s.nnz_kind, s.nnz_a, s.nnz_b = NNZ_UNIFORM, float(nnz[1]), float(nnz[2])
    elif nnz[0] == "poisson":
        s.nnz_kind, s.nnz_a, s.nnz_b = NNZ_POISSON, float(nnz[1]), 0.0
        s.nnz_min = int(nnz[2])
    elif nnz[0] == "lognormal":
        s.nnz_kind, s.nnz_a, s.nnz_b = NNZ_LOGNORMAL, float(nnz[1]), float(nnz[2])
        s.nnz_min, s.nnz_max = int(nnz[3]), int(nnz[4])
    else:
        raise ValueError(nnz)
    if idx[0] == "uniform":
        s.idx_kind, s.zipf_s = IDX_UNIFORM, 0.0
    elif idx[0] == "zipf":
        s.idx_kind, s.zipf_s = IDX_ZIPF, float(idx[1])
    else:
        raise ValueError(idx)
    s.val_kind = int(val)
    nt = n_threads or _threads()
    lens = np.zeros(n_rows, dtype=np.int32)
    fe = None
    if force_empty is not None:
        fe = np.ascontiguousarray(force_empty, dtype=np.uint8)
        assert fe.shape == (n_rows,)
    tot = lib.synth_row_nnz(ctypes.byref(s), fe.ctypes.data if fe is not None else None,
                            lens.ctypes.data, nt)
    if tot < 0:
        raise OverflowError("nnz exceeds 2^31-1")
    indptr = np.zeros(n_rows + 1, dtype=np.int64)
    np.cumsum(lens, out=indptr[1:])
    indptr = indptr.astype(np.int32)
    indices = np.empty(int(tot), dtype=np.int32)
    values = np.empty(int(tot), dtype=np.float32)
    rc = lib.synth_fill(ctypes.byref(s), indptr.ctypes.data, indices.ctypes.data,
                        values.ctypes.data, nt)
    if rc != 0:
        raise MemoryError("synth_fill failed")
    return HostCSR(indptr, indices, values, n_rows, dim)


def subset(seed: int, matrix: int, n: int, k: int) -> np.ndarray:
    """k distinct ids from range(n): a seeded partial Fisher-Yates shuffle."""
    out = np.empty(k, dtype=np.int64)
    if _load().synth_subset(seed, matrix, n, k, out.ctypes.data) != 0:
        raise ValueError("bad subset request")
    return out


def philox4x32_10(ctr, key):
    c = np.asarray(ctr, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    o = np.zeros(4, dtype=np.uint32)
    _load().synth_philox4x32_10(c.ctypes.data, k.ctypes.data, o.ctypes.data)
    return o


# ---------------------------------------------------------------------------
# The five workloads. Config "pages" is the production shape of §1 of the page.
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    n_query: int
    n_item: int
    dim: int
    chunk_size: int
    seed: int
    nnz: tuple
    idx: tuple
    val: int
    empty_item_frac: float = 0.0
    queries_from_items: bool = False
    description: str = ""


WORKLOADS = {
    "tiny": Workload("tiny", 256, 4096, 65536, 4096, 0, ("uniform", 8, 32), ("uniform",),
                     VAL_LOGNORMAL,
                     description="256 x 4096, dim 65536, nnz U{8..32}, uniform ids, lognormal"),
    "mid": Workload("mid", 2000, 100000, 500000, 8192, 1, ("poisson", 43, 1), ("zipf", 1.1),
                    VAL_LOGNORMAL,
                    description="2000 x 100000, dim 500000, Poisson(43)>=1, Zipf(1.1), lognormal"),
    "pages": Workload("pages", 50000, 2000000, 1200000, 8192, 2, ("poisson", 43, 1),
                      ("zipf", 1.1), VAL_LOGNORMAL,
                      description="50000 x 2000000, dim 1.2M, Poisson(43)>=1, Zipf(1.1), "
                                  "lognormal; rotating 50000x8192 output, row sums per chunk"),
    "dense": Workload("dense", 20000, 500000, 30522, 8192, 3, ("poisson", 120, 0),
                      ("zipf", 1.0), VAL_LOG1P_HALFNORMAL,
                      description="20000 x 500000, dim 30522, Poisson(120), Zipf(1.0), "
                                  "log1p(|N(0,1)|) (zeros redrawn)"),
    "edge": Workload("edge", 10000, 1000000, 1200000, 8192, 4,
                     ("lognormal", 3.5, 1.2, 0, 2000), ("uniform",), VAL_NORMAL,
                     empty_item_frac=0.01, queries_from_items=True,
                     description="10000 x 1000000, dim 1.2M, nnz clip(rint(LN(3.5,1.2)),0,2000), "
                                 "1% items empty, N(0,1) signed, queries = random item subset"),
}
WORKLOAD_ORDER = ["tiny", "mid", "pages", "dense", "edge"]


def make_items(w: Workload, n_item: int | None = None) -> HostCSR:
    n = w.n_item if n_item is None else n_item
    fe = None
    if w.empty_item_frac > 0:
        k = int(round(w.empty_item_frac * n))
        fe = np.zeros(n, dtype=np.uint8)
        fe[subset(w.seed, 0, n, k)] = 1
    return make_corpus(n, w.dim, w.seed, 0, nnz=w.nnz, idx=w.idx, val=w.val, force_empty=fe)


def make_workload(w: Workload | str, n_item: int | None = None, n_query: int | None = None):
    """Return (queries, items, extra) host CSRs for a workload.

    extra["query_item"] holds, for workloads whose queries are item copies,
    the item id each query row was copied from.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    items = make_items(w, n_item)
    nq = w.n_query if n_query is None else n_query
    extra = {}
    if w.queries_from_items:
        perm = subset(w.seed, 1, items.n_rows, nq)
        queries = items.take_rows(perm)
        extra["query_item"] = perm
    else:
        queries = make_corpus(nq, w.dim, w.seed, 1, nnz=w.nnz, idx=w.idx, val=w.val)
    return queries, items, extra
