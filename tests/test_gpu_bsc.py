"""The Block-Sparse CSR codec of §3.2 of "稀疏嵌入批量相似度计算的工程化实践"
on the GPU against the oracle codec (oracle/bsc.py), through the C ABI.

Encoding is integer work: the GPU's row byte pointers, varint bytes and
packed offsets must equal the oracle's byte for byte (whole streams up to a
few million entries; at the full pages size the whole byte-pointer array and
eight windows of rows). Decoding must give back the CSR's column indices
exactly, and a corpus prepared from its Block-Sparse form must score as the
CSR-prepared one, bit for bit. Malformed encodings are reported, never
faulted on.
"""
import os
import sys

import numpy as np
import pytest

import synth
from oracle import bsc
from test_oracle_bsc import random_csr

pytestmark = pytest.mark.gpu

# the widest matrix the library takes (sizes below 2^31 - 1): columns to 2^31 - 3,
# block ids to 2^21 - 1, three-byte varints
N_COLS_MAX = 2 ** 31 - 2


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_embedding_exact_amd as sps
    sps.load_library()
    return torch, sps, torch.device("cuda:0")


def report(line):
    print("\n[parity] " + line, file=sys.stderr, flush=True)
    path = os.environ.get("SPS_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write("[parity] " + line + "\n")


class _M:
    def __init__(self, indptr, indices, n_cols, values=None):
        self.indptr = np.asarray(indptr, dtype=np.int32)
        self.indices = np.asarray(indices, dtype=np.int32)
        self.values = np.ones(self.indices.size, np.float32) if values is None else values
        self.n_rows, self.n_cols = self.indptr.size - 1, int(n_cols)


def _gpu_encode(env, m):
    torch, sps, dev = env
    b = sps.bsc_encode(sps.CSR.from_host(m, dev))
    torch.cuda.synchronize()
    return b, b.bptr.cpu().numpy(), b.blocks.cpu().numpy(), b.offsets.cpu().numpy()


def _check_whole(env, name, m):
    torch, sps, dev = env
    b, bp, bl, of = _gpu_encode(env, m)
    rb, rl, ro = bsc.encode(m.indptr, m.indices)
    assert np.array_equal(bp, rb), name
    assert np.array_equal(bl, rl), name
    assert of.size % 4 == 0 and of.size - ro.size < 4
    assert np.array_equal(of[:ro.size], ro) and not of[ro.size:].any(), name
    dec = sps.bsc_decode(b)
    assert np.array_equal(dec.indices.cpu().numpy(), m.indices), name
    return b


def test_encode_decode_workloads(env):
    sizes = {"tiny": {}, "mid": {}, "edge": {"n_item": 50000, "n_query": 10},
             "dense": {"n_item": 20000, "n_query": 10}}
    for name, kw in sizes.items():
        q, items, _ = synth.make_workload(name, **kw)
        b = _check_whole(env, name, items)
        csr_bytes = 4 * items.nnz
        report("bsc %s items %d x %d: encode = oracle byte for byte, decode exact; index bytes "
               "%.2f per entry (CSR 4.00)" % (name, items.n_rows, items.n_cols,
                                               b.index_bytes() / max(items.nnz, 1)))
        assert b.index_bytes() < csr_bytes + 4 * (items.n_rows + 1) + 8


def test_encode_decode_edges(env):
    """Up to the largest column the library takes (three-byte varints), rows spanning several
    64-byte windows with values straddling them, empty rows, an empty matrix."""
    cases = {
        "int32 range": random_csr(6, 300, N_COLS_MAX, 200),
        "ragged": random_csr(7, 777, 1024 * 300, 700, empty_frac=0.3),
        "tiny dims": random_csr(8, 50, 3, 3),
    }
    rng = np.random.default_rng(3)
    wide = np.sort(rng.choice(N_COLS_MAX, 1000, replace=False))
    cases["one long row"] = (np.array([0, 0, 1000, 1000]), wide)
    cases["all empty"] = (np.zeros(9, np.int64), np.zeros(0, np.int64))
    for name, (indptr, idx) in cases.items():
        n_cols = N_COLS_MAX if name in ("int32 range", "one long row") else \
            (1024 * 300 if name in ("ragged", "all empty") else 3)
        _check_whole(env, name, _M(indptr, idx, n_cols))
    report("bsc edge cases (int32 columns, 1000-entry row over 30 windows, empty rows, "
           "nnz 0): exact")


def test_pages_full_size(env):
    """The benchmark's item corpus (2M rows, 86M entries)."""
    torch, sps, dev = env
    q, items, _ = synth.make_workload("pages")
    b, bp, bl, of = _gpu_encode(env, items)
    ip = items.indptr.astype(np.int64)
    # whole byte-pointer array: one byte per difference, one more from 2^7, 2^14, 2^21
    blk = items.indices.astype(np.int64) // 1024
    prev = np.zeros_like(blk)
    prev[1:] = blk[:-1]
    prev[ip[:-1][np.diff(ip) > 0]] = 0
    dlt = blk - prev
    nb = 1 + (dlt >= 128).astype(np.int64) + (dlt >= 16384) + (dlt >= 2 ** 21)
    ref_bptr = np.concatenate([[0], np.cumsum(nb)])[ip]
    assert np.array_equal(bp.astype(np.int64), ref_bptr)
    # eight windows of 3000 rows, each starting at an entry that is a multiple of 4
    # (40 bits: its offsets start on a byte)
    rng = np.random.default_rng(21)
    for r0 in rng.choice(items.n_rows - 3000, 8, replace=False):
        while ip[r0] % 4:
            r0 += 1
        r1 = r0 + 3000
        e0, e1 = int(ip[r0]), int(ip[r1])
        sb, sl, so = bsc.encode(ip[r0:r1 + 1] - e0, items.indices[e0:e1])
        assert np.array_equal(bp[r0:r1 + 1] - bp[r0], sb)
        assert np.array_equal(bl[bp[r0]:bp[r1]], sl)
        o0, full = 10 * e0 // 8, (10 * (e1 - e0)) // 8
        assert np.array_equal(of[o0:o0 + full], so[:full])
        rem = (10 * (e1 - e0)) % 8
        if rem:
            assert (of[o0 + full] & ((1 << rem) - 1)) == so[full]
    dec = sps.bsc_decode(b)
    assert torch.equal(dec.indices, torch.as_tensor(items.indices, device=dev))
    # a corpus prepared from the Block-Sparse form scores as the CSR-prepared one
    it_c = sps.prepare(sps.CSR.from_host(items, dev), chunk_size=8192)
    it_b = sps.prepare(b, chunk_size=8192)
    qq_c = sps.prepare_queries(sps.CSR.from_host(q, dev), it_c)
    qq_b = sps.prepare_queries(sps.CSR.from_host(q, dev), it_b)
    o1 = torch.empty(q.n_rows, 8192, dtype=torch.float32, device=dev)
    o2 = torch.empty_like(o1)
    for c in (0, it_c.num_chunks - 1):
        sps.cosine_chunk(qq_c, it_c, c, o1)
        sps.cosine_chunk(qq_b, it_b, c, o2)
        n = it_c.chunk_len(c)
        assert torch.equal(o1[:, :n], o2[:, :n])
    report("bsc pages items 2Mx1.2M (86M entries): bptr = oracle; 8 windows of 3000 rows "
           "= oracle byte for byte; decode exact; scores from the decoded corpus bit-equal; "
           "index bytes %.3f per entry (CSR 4)" % (b.index_bytes() / items.nnz))


def test_malformed_and_errors(env):
    torch, sps, dev = env
    q, items, _ = synth.make_workload("tiny")
    b, bp, bl, of = _gpu_encode(env, items)
    # continuation bits everywhere: no value ends
    bad = sps.BSC(b.indptr, b.bptr, b.blocks | 0x80, b.offsets, b.values, b.n_rows, b.n_cols)
    with pytest.raises(sps.SpsError):
        sps.bsc_decode(bad)
    # a row's byte range shifted by one, byte pointers out of order and out of range
    for k, v in ((5, 1), (5, -3), (7, 10 ** 6)):
        bp2 = b.bptr.clone()
        bp2[k] += v
        with pytest.raises(sps.SpsError):
            sps.bsc_decode(sps.BSC(b.indptr, bp2, b.blocks, b.offsets, b.values, b.n_rows,
                                   b.n_cols))
    # the well-formed one still decodes
    assert np.array_equal(sps.bsc_decode(b).indices.cpu().numpy(), items.indices)
    # a non-canonical CSR is refused by the encoder
    m = _M([0, 3], [5, 2, 9], 10)
    with pytest.raises(sps.SpsError):
        sps.bsc_encode(sps.CSR.from_host(m, dev))
    # a too small offset buffer and misaligned sizes are refused
    c = sps.CSR.from_host(items, dev)._c()
    import ctypes
    ok = sps._lib.sps_bsc_encode(ctypes.byref(c), b.bptr.data_ptr(), b.blocks.data_ptr(),
                                 b.blocks.numel(), b.offsets.data_ptr(), b.offsets.numel() - 4,
                                 None)
    assert ok == -4


def _rows_of_lengths(seed, lengths, n_cols):
    """A canonical CSR whose rows have the given lengths (sorted distinct columns)."""
    rng = np.random.default_rng(seed)
    rows = [np.sort(rng.choice(n_cols, int(n), replace=False)) for n in lengths]
    indptr = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    idx = np.concatenate(rows) if rows else np.zeros(0, np.int64)
    return indptr, idx.astype(np.int32)


def test_decode_paths_and_alignment(env):
    """The decoder takes a wave's rows one per lane with the indices gathered in LDS when the
    wave's rows are all short (at most 256 entries) and span at most 3072 entries; one per
    lane with direct stores when they span more; and rows of more than 256 entries with the
    whole wave. Each path, on varint and offset buffers that start 0 to 3 bytes past a
    4-byte boundary (the decoder reads whole aligned words only inside the buffers)."""
    torch, sps, dev = env
    n_cols = 1024 * 1000
    cases = {
        # every wave staged: 64 rows x 40 entries = 2560 per wave
        "staged": [40] * 640,
        # one lane per row, direct stores: 64 x 60 = 3840 entries per wave
        "direct": [60] * 200,
        # lengths about the 256-entry boundary: waves with rows for the whole wave
        "mixed": [0, 1, 5, 43, 100, 255, 256, 257, 300, 3, 2] * 30,
    }
    for name, lengths in cases.items():
        indptr, idx = _rows_of_lengths(11, lengths, n_cols)
        m = _M(indptr, idx, n_cols)
        b, bp, bl, of = _gpu_encode(env, m)
        for shift in (0, 1, 2, 3):
            # the same bytes at a buffer position that is `shift` past a word boundary
            big_b = torch.zeros(bl.size + 8, dtype=torch.uint8, device=dev)
            big_o = torch.zeros(of.size + 8, dtype=torch.uint8, device=dev)
            big_b[shift:shift + bl.size] = b.blocks
            big_o[shift:shift + of.size] = b.offsets
            sb = big_b[shift:shift + bl.size]
            so = big_o[shift:shift + of.size]
            assert sb.data_ptr() % 4 == shift % 4 or big_b.data_ptr() % 4 != 0
            dec = sps.bsc_decode(sps.BSC(b.indptr, b.bptr, sb, so, b.values, b.n_rows, b.n_cols))
            assert np.array_equal(dec.indices.cpu().numpy(), idx), (name, shift)
    report("bsc decode paths: staged (64 x 40), direct (64 x 60), rows 0..300 entries about the "
           "256 boundary; buffers at byte offsets 0..3: exact")
