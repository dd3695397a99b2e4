"""Pins of the Block-Sparse CSR codec oracle (oracle/bsc.py) to things other
than itself: a worked example computed by hand (tests/golden), protobuf's
varint encoder (the same unsigned base-128 form), numpy's little-endian bit
packing, closed-form sizes, and round trips over random canonical CSR up to
the largest int32 column. Planted mistakes must each fail one of them.

The format is that of §3.2 of "稀疏嵌入批量相似度计算的工程化实践".
"""
import json
import os

import numpy as np
import pytest

from oracle import bsc

HERE = os.path.dirname(os.path.abspath(__file__))


def golden():
    with open(os.path.join(HERE, "golden", "bsc_worked_example.json")) as f:
        return json.load(f)


def random_csr(seed, n_rows, n_cols, max_nnz, empty_frac=0.1):
    rng = np.random.default_rng(seed)
    counts = rng.integers(0, max_nnz + 1, n_rows)
    counts[rng.random(n_rows) < empty_frac] = 0
    counts = np.minimum(counts, n_cols)
    rows = []
    for c in counts:
        # clustered low dims and a few anywhere, like dictionary-prefix data
        k_lo = int(c) // 2
        lo = rng.choice(min(n_cols, 50_000), min(k_lo, min(n_cols, 50_000)), replace=False)
        hi = rng.integers(0, n_cols, int(c) - k_lo)
        rows.append(np.unique(np.concatenate([lo, hi]).astype(np.int64)))
    indptr = np.zeros(n_rows + 1, dtype=np.int64)
    indptr[1:] = np.cumsum([len(r) for r in rows])
    idx = np.concatenate(rows) if rows else np.zeros(0, np.int64)
    return indptr, idx.astype(np.int32)


def pin_worked_example():
    g = golden()
    for enc in (bsc.encode_loop, bsc.encode):
        bptr, blocks, offsets = enc(g["indptr"], g["indices"])
        assert bptr.tolist() == g["bptr"]
        assert blocks.tobytes().hex() == g["blocks_hex"]
        assert offsets.tobytes().hex() == g["offsets_hex"]
    blocks = np.frombuffer(bytes.fromhex(g["blocks_hex"]), dtype=np.uint8)
    offsets = np.frombuffer(bytes.fromhex(g["offsets_hex"]), dtype=np.uint8)
    for dec in (bsc.decode_loop, bsc.decode):
        assert dec(g["indptr"], g["bptr"], blocks, offsets).tolist() == g["indices"]


def pin_varint_is_protobufs():
    from google.protobuf.internal.encoder import _VarintBytes
    vals = [0, 1, 127, 128, 255, 300, 16383, 16384, 2097151, 2097152, 2 ** 31 - 1]
    for v in vals:
        assert bsc.varint(v) == _VarintBytes(v), v
    # one row whose differences are exactly vals: its byte stream is theirs
    blocks = np.cumsum(vals[:-1])
    idx = blocks * bsc.BLOCK + 7
    _, stream, _ = bsc.encode([0, len(idx)], idx)
    assert stream.tobytes() == b"".join(_VarintBytes(v) for v in vals[:-1])


def pin_offsets_are_little_endian_bits():
    indptr, idx = random_csr(3, 50, 2 ** 31 - 1, 40)
    off = idx.astype(np.int64) % bsc.BLOCK
    bits = ((off[:, None] >> np.arange(bsc.OFFSET_BITS)) & 1).astype(np.uint8).ravel()
    ref = np.packbits(bits, bitorder="little")
    for enc in (bsc.encode_loop, bsc.encode):
        _, _, packed = enc(indptr, idx)
        assert np.array_equal(packed, ref)


def pin_sizes():
    indptr, idx = random_csr(4, 200, 1_200_000, 60)
    bptr, blocks, offsets = bsc.encode(indptr, idx)
    assert offsets.size == (10 * idx.size + 7) // 8 == bsc.offsets_nbytes(idx.size)
    # the bytes of a row: one per difference, one more from 2^7, 2^14, 2^21
    for r in range(len(indptr) - 1):
        blk = idx[indptr[r]:indptr[r + 1]].astype(np.int64) // 1024
        d = np.diff(np.concatenate([[0], blk]))
        assert np.all(d >= 0)
        n = int(np.sum(1 + (d >= 128) + (d >= 16384) + (d >= 2 ** 21)))
        assert bptr[r + 1] - bptr[r] == n
    assert bptr[-1] == blocks.size


def pin_round_trips():
    cases = [random_csr(5, 300, 1_200_000, 90), random_csr(6, 100, 2 ** 31 - 1, 30),
             random_csr(7, 40, 1024, 1024, empty_frac=0.3), random_csr(8, 5, 3, 3),
             (np.zeros(4, np.int64), np.zeros(0, np.int32))]
    for indptr, idx in cases:
        e1 = bsc.encode_loop(indptr, idx)
        e2 = bsc.encode(indptr, idx)
        for a, b in zip(e1, e2):
            assert np.array_equal(a, b)
        assert np.array_equal(bsc.decode_loop(indptr, *e1), idx)
        assert np.array_equal(bsc.decode(indptr, *e2), idx)


ALL_PINS = [pin_worked_example, pin_varint_is_protobufs, pin_offsets_are_little_endian_bits,
            pin_sizes, pin_round_trips]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin()


MUTANTS = {1: "differences not restarted at a row start",
           2: "most significant 7-bit group first",
           3: "offset bits packed most significant first"}


@pytest.mark.parametrize("k", sorted(MUTANTS))
def test_mutant_is_caught(k, monkeypatch):
    monkeypatch.setattr(bsc, "_MUTANT", k)
    failed = []
    for pin in ALL_PINS:
        try:
            pin()
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "mutant %d (%s) passed every pin" % (k, MUTANTS[k])


def test_large_random_numpy_round_trip():
    """The numpy codec at a size the loop version cannot reach."""
    rng = np.random.default_rng(11)
    n_rows, n_cols = 20_000, 1_200_000
    counts = rng.poisson(43, n_rows)
    indptr = np.zeros(n_rows + 1, np.int64)
    indptr[1:] = np.cumsum(counts)
    idx = np.concatenate([np.sort(rng.choice(n_cols, c, replace=False)) for c in counts])
    e = bsc.encode(indptr, idx)
    assert np.array_equal(bsc.decode(indptr, *e), idx)
