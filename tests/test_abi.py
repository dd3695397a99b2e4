"""The C ABI without a GPU: the library loads, exports every declared symbol,
and its host-side argument checks return the documented statuses."""
import ctypes
import os
import re

import pytest

import sparse_embedding_exact_amd as sps

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "sps.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sps_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return sps.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_symbols()
    assert len(names) >= 15
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert set(names) == set(sps.SIGNATURES), set(names) ^ set(sps.SIGNATURES)


def test_status_strings(lib):
    for code in range(0, -9, -1):
        s = lib.sps_status_string(code)
        assert s and s != b"unknown status"
    assert lib.sps_status_string(-99) == b"unknown status"


def test_items_sizing(lib):
    p, s = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.sps_items_workspace_size(2_000_000, 1_200_000, 86_000_000, 8192,
                                        ctypes.byref(p), ctypes.byref(s)) == 0
    # dim index: 1960 slices, up to 2 x nnz + slices 16-byte buckets; postings: 8 B each
    assert p.value >= (2 * 86_000_000 + 1960) * 16 + 86_000_000 * 8
    assert p.value < 4 * 86_000_000 * 16  # no per-slice col_ptr[dim + 1]
    assert s.value >= 86_000_000 * 10
    assert p.value % 256 == 0 and s.value % 256 == 0
    bad = [(-1, 10, 0, 8192), (10, 0, 0, 8192), (10, 10, 0, 0), (10, 10, 0, (1 << 20) + 1),
           (10, 10, -5, 8192)]
    for a in bad:
        assert lib.sps_items_workspace_size(*a, ctypes.byref(p), ctypes.byref(s)) == -1, a
    assert lib.sps_items_workspace_size(2**31, 10, 0, 8192, ctypes.byref(p),
                                        ctypes.byref(s)) == -6
    assert lib.sps_items_workspace_size(10, 10, 0, 8192, None, ctypes.byref(s)) == -1
    assert b"NULL" in lib.sps_last_error_message()


def test_null_handles_rejected(lib):
    out = ctypes.c_void_p()
    assert lib.sps_prepare(None, 8192, None, 0, None, 0, None, ctypes.byref(out)) == -1
    assert lib.sps_prepare_queries(None, None, None, 0, None, ctypes.byref(out)) == -1
    assert lib.sps_cosine_chunk(None, None, 0, None, 8192, None, None) == -1
    assert lib.sps_cosine_stream(None, None, 0, 1, None, 8192, None, None) == -1
    assert lib.sps_items_info(None, None, None, None, None, None) == -1
    assert lib.sps_queries_inv_norms(None, None) == -1
    size = ctypes.c_size_t()
    assert lib.sps_queries_workspace_size(None, 10, 10, 10, ctypes.byref(size)) == -1
    assert lib.sps_row_inv_norms(None, None, None) == -1
    assert lib.sps_validate_csr(None, None, None, None, None) == -1
    assert lib.sps_cosine_stream_host(None, None, 0, 1, None, 8192, None, None, 8192, None,
                                      None, None) == -1
    assert lib.sps_cosine_chunk_threshold(None, None, 0, 0.5, None, 0, None, None, None) == -1
    assert lib.sps_bsc_decode(None, None, None, None) == -1
    assert lib.sps_bsc_encode_sizes(None, None, None, None, None) == -1
    assert lib.sps_bsc_encode(None, None, None, 0, None, 0, None) == -1
    lib.sps_items_destroy(None)
    lib.sps_queries_destroy(None)


def test_bsc_offset_sizing(lib):
    """ceil(10 nnz / 8) bytes of 10-bit offsets, rounded up to whole 32-bit words."""
    n = ctypes.c_size_t()
    for nnz, want in ((0, 0), (1, 4), (3, 4), (4, 8), (8, 12), (16, 20), (85_991_513, 107_489_392)):
        assert lib.sps_bsc_offsets_bytes(nnz, ctypes.byref(n)) == 0
        assert n.value == want, nnz
    assert lib.sps_bsc_offsets_bytes(-1, ctypes.byref(n)) == -1
    assert lib.sps_bsc_offsets_bytes(5, None) == -1


def test_csr_shape_checks(lib):
    out = ctypes.c_void_p()
    c = sps._Csr(10, 100, 5, 0x1000, 0x2000, 0x3000)
    # workspace NULL after a valid shape -> invalid argument, before any device work
    assert lib.sps_prepare(ctypes.byref(c), 8192, None, 0, None, 0, None, ctypes.byref(out)) == -1
    c = sps._Csr(10, 0, 5, 0x1000, 0x2000, 0x3000)
    assert lib.sps_prepare(ctypes.byref(c), 8192, None, 0, None, 0, None, ctypes.byref(out)) == -1
    c = sps._Csr(10, 100, 5, 0x1000, None, 0x3000)
    assert lib.sps_prepare(ctypes.byref(c), 8192, None, 0, None, 0, None, ctypes.byref(out)) == -1
    c = sps._Csr(2**31, 100, 5, 0x1000, 0x2000, 0x3000)
    assert lib.sps_prepare(ctypes.byref(c), 8192, None, 0, None, 0, None, ctypes.byref(out)) == -6
    # too-small workspace is reported before any device work
    c = sps._Csr(10, 100, 5, 0x1000, 0x2000, 0x3000)
    assert lib.sps_prepare(ctypes.byref(c), 8192, 0x10000, 16, 0x20000, 16, None,
                           ctypes.byref(out)) == -4
    assert out.value is None
