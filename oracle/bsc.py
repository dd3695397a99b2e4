"""Block-Sparse CSR codec, oracle side (plain Python and numpy).

TEST INFRASTRUCTURE. Only ``tests/`` may import this module; the GPU library
never imports or calls it, and it imports nothing from the GPU library.

The format follows §3.2 of the page "稀疏嵌入批量相似度计算的工程化实践". A
column index d is split into the pair (block id, local offset) with block
size B = 1024: block = d // B, offset = d % B. The block ids of a row are
sorted (a canonical CSR row is), stored as differences from the previous
entry's block id, and each difference is written as a variable-length integer
(one byte for small differences, two or three for large ones). The local
offsets take 10 bits each, packed back to back. Values stay float32, and a
row pointer locates each row's entries.

Readings where the page leaves a point open or garbled (each one is shared
by the GPU codec):

* the first difference of a row is taken from 0, so that rows decode
  independently of each other;
* the variable-length integer is the unsigned base-128 form: 7 value bits
  per byte, least significant group first, the high bit set on every byte of
  a value except its last;
* since those bytes cannot be located with the entry pointer, a second row
  pointer ``bptr`` (int32, n_rows + 1) gives the byte position of each row's
  block-id bytes; ``indptr`` (the CSR's) still locates offsets and values;
* the 10-bit offsets are packed over the whole matrix in entry order,
  least significant bit first: entry k occupies bits 10k .. 10k + 9 of the
  stream, and byte j holds bits 8j .. 8j + 7 with bit 8j in its lowest place
  (the page's "8 offsets per byte" is read as 8 offsets per 10 bytes).

Two implementations: the ``*_loop`` functions, one entry at a time in pure
Python (small inputs), and ``encode`` / ``decode``, the same steps on whole
numpy arrays (any size). Pins in tests/test_oracle_bsc.py.
"""
from __future__ import annotations

import numpy as np

BLOCK = 1024
OFFSET_BITS = 10

# a planted mistake, for tests/test_oracle_bsc.py only (0 = none):
# 1 differences not restarted at a row start, 2 most significant 7-bit group
# first, 3 offset bits packed most significant first
_MUTANT = 0


def offsets_nbytes(nnz: int) -> int:
    """Bytes of the packed offset stream: ceil(10 nnz / 8)."""
    return (OFFSET_BITS * int(nnz) + 7) // 8


def varint(v: int) -> bytes:
    """Unsigned base-128 bytes of v >= 0."""
    assert v >= 0
    groups = []
    while True:
        groups.append(v & 0x7F)
        v >>= 7
        if v == 0:
            break
    if _MUTANT == 2:
        groups.reverse()
    return bytes([g | 0x80 for g in groups[:-1]] + [groups[-1]])


def encode_loop(indptr, indices):
    """(bptr int32[n_rows + 1], block bytes uint8, offset bytes uint8) of a CSR."""
    indptr = [int(x) for x in indptr]
    indices = [int(x) for x in indices]
    n_rows, nnz = len(indptr) - 1, len(indices)
    out = bytearray()
    bptr = [0]
    prev = 0
    for r in range(n_rows):
        if _MUTANT != 1:
            prev = 0
        for k in range(indptr[r], indptr[r + 1]):
            b = indices[k] // BLOCK
            out += varint(b - prev)
            prev = b
        bptr.append(len(out))
    packed = bytearray(offsets_nbytes(nnz))
    for k, d in enumerate(indices):
        off = d % BLOCK
        for i in range(OFFSET_BITS):
            bit = (off >> (OFFSET_BITS - 1 - i if _MUTANT == 3 else i)) & 1
            pos = OFFSET_BITS * k + i
            packed[pos // 8] |= bit << (pos % 8)
    return (np.array(bptr, dtype=np.int32), np.frombuffer(bytes(out), dtype=np.uint8).copy(),
            np.frombuffer(bytes(packed), dtype=np.uint8).copy())


def decode_loop(indptr, bptr, blocks, offsets):
    """int32 column indices from the three streams (checks that every row's
    bytes hold exactly its entries)."""
    indptr = [int(x) for x in indptr]
    bptr = [int(x) for x in bptr]
    blocks = bytes(np.asarray(blocks, dtype=np.uint8))
    offsets = bytes(np.asarray(offsets, dtype=np.uint8))
    n_rows = len(indptr) - 1
    cols = []
    for r in range(n_rows):
        p, end = bptr[r], bptr[r + 1]
        prev = 0
        for k in range(indptr[r], indptr[r + 1]):
            v, shift = 0, 0
            while True:
                byte = blocks[p]
                p += 1
                v |= (byte & 0x7F) << shift
                shift += 7
                if byte < 0x80:
                    break
            prev += v
            off = 0
            for i in range(OFFSET_BITS):
                pos = OFFSET_BITS * k + i
                off |= ((offsets[pos // 8] >> (pos % 8)) & 1) << i
            cols.append(prev * BLOCK + off)
        assert p == end, "row %d: %d block bytes for its entries, %d stored" % (r, p - bptr[r],
                                                                               end - bptr[r])
    return np.array(cols, dtype=np.int32)


def _row_of_entry(indptr: np.ndarray) -> np.ndarray:
    return np.repeat(np.arange(len(indptr) - 1, dtype=np.int64), np.diff(indptr))


def encode(indptr, indices):
    """``encode_loop`` on whole arrays."""
    indptr = np.asarray(indptr, dtype=np.int64)
    d = np.asarray(indices, dtype=np.int64)
    nnz = d.size
    blk = d // BLOCK
    off = d % BLOCK
    # previous entry's block id, 0 at the start of every row
    prev = np.zeros(nnz, dtype=np.int64)
    prev[1:] = blk[:-1]
    if _MUTANT != 1:
        first = indptr[:-1][np.diff(indptr) > 0]
        prev[first] = 0
    delta = blk - prev
    nb = np.ones(nnz, dtype=np.int64)
    for j in range(1, 5):
        nb += delta >= (1 << (7 * j))
    start = np.zeros(nnz + 1, dtype=np.int64)
    np.cumsum(nb, out=start[1:])
    out = np.zeros(int(start[-1]), dtype=np.uint8)
    for j in range(int(nb.max()) if nnz else 0):
        m = nb > j
        shift = 7 * (nb[m] - 1 - j) if _MUTANT == 2 else 7 * j
        byte = (delta[m] >> shift) & 0x7F
        byte |= np.where(nb[m] > j + 1, 0x80, 0)
        out[start[:-1][m] + j] = byte.astype(np.uint8)
    bptr = start[indptr].astype(np.int32)
    packed = np.zeros(offsets_nbytes(nnz) + 1, dtype=np.int64)
    if _MUTANT == 3:
        off = np.array([int("{:010b}".format(int(x))[::-1], 2) for x in off], dtype=np.int64)
    bit = OFFSET_BITS * np.arange(nnz, dtype=np.int64)
    w = off << (bit % 8)  # up to 17 bits, spread over three bytes from byte bit // 8
    # bit // 8 = floor(10k / 8) differs for different entries k, so within one
    # of the three assignments below no byte is named twice
    for i in range(3):
        packed[bit // 8 + i] |= (w >> (8 * i)) & 0xFF
    return bptr, out, packed[:offsets_nbytes(nnz)].astype(np.uint8)


def decode(indptr, bptr, blocks, offsets):
    """``decode_loop`` on whole arrays."""
    indptr = np.asarray(indptr, dtype=np.int64)
    bptr = np.asarray(bptr, dtype=np.int64)
    b = np.asarray(blocks, dtype=np.uint8).astype(np.int64)
    nnz = int(indptr[-1])
    last = (b & 0x80) == 0                       # the last byte of each value
    n_vals = int(last.sum())
    assert n_vals == nnz, "%d values in the block bytes for %d entries" % (n_vals, nnz)
    # value index of every byte, and its place within the value
    vid = np.zeros(b.size, dtype=np.int64)
    vid[1:] = np.cumsum(last)[:-1]
    vstart = np.zeros(nnz + 1, dtype=np.int64)
    vstart[1:] = np.nonzero(last)[0] + 1
    place = np.arange(b.size, dtype=np.int64) - vstart[vid]
    delta = np.zeros(nnz, dtype=np.int64)
    np.add.at(delta, vid, (b & 0x7F) << (7 * place))
    # every row's bytes hold exactly its values
    assert np.array_equal(vstart[indptr], bptr), "row byte pointers disagree with the values"
    # block ids: the differences summed from each row's start
    cs = np.cumsum(delta)
    row = _row_of_entry(indptr)
    base = np.concatenate([[0], cs])[indptr[:-1]]
    blk = cs - base[row]
    o = np.concatenate([np.asarray(offsets, dtype=np.uint8).astype(np.int64), [0, 0]])
    bit = OFFSET_BITS * np.arange(nnz, dtype=np.int64)
    w = o[bit // 8] | (o[bit // 8 + 1] << 8) | (o[bit // 8 + 2] << 16)
    off = (w >> (bit % 8)) & (BLOCK - 1)
    return (blk * BLOCK + off).astype(np.int32)
