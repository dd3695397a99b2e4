"""The seeded input generator: determinism, canonical CSR, workload shapes."""
import numpy as np

import synth


def _canonical(m):
    assert m.indptr[0] == 0 and m.indptr[-1] == len(m.indices) == len(m.values)
    assert np.all(np.diff(m.indptr) >= 0)
    assert m.indices.min(initial=0) >= 0 and m.indices.max(initial=0) < m.n_cols
    same_row = np.repeat(np.arange(m.n_rows), np.diff(m.indptr))
    step = np.diff(m.indices.astype(np.int64))
    inside = same_row[1:] == same_row[:-1]
    assert np.all(step[inside] > 0), "indices not strictly ascending within rows"
    assert np.all(np.isfinite(m.values))


def test_philox_known_answers():
    # Known-answer vectors of Philox4x32-10 (Salmon et al., SC'11, Random123 KAT)
    assert [hex(x) for x in synth.philox4x32_10([0, 0, 0, 0], [0, 0])] == \
        ['0x6627e8d5', '0xe169c58d', '0xbc57ac4c', '0x9b00dbd8']
    assert [hex(x) for x in synth.philox4x32_10([0xffffffff] * 4, [0xffffffff] * 2)] == \
        ['0x408f276d', '0x41c83b0e', '0xa20bc7c6', '0x6d5451fd']


def test_deterministic_and_thread_independent():
    w = synth.WORKLOADS["mid"]
    a = synth.make_corpus(3000, w.dim, 7, 0, nnz=w.nnz, idx=w.idx, val=w.val, n_threads=1)
    b = synth.make_corpus(3000, w.dim, 7, 0, nnz=w.nnz, idx=w.idx, val=w.val, n_threads=5)
    for x, y in [(a.indptr, b.indptr), (a.indices, b.indices), (a.values, b.values)]:
        assert np.array_equal(x, y)
    c = synth.make_corpus(3000, w.dim, 8, 0, nnz=w.nnz, idx=w.idx, val=w.val)
    assert not np.array_equal(a.indices[:100], c.indices[:100])


def test_tiny_shape():
    q, i, _ = synth.make_workload("tiny")
    assert (q.n_rows, i.n_rows, i.n_cols) == (256, 4096, 65536)
    for m in (q, i):
        _canonical(m)
        lens = np.diff(m.indptr)
        assert lens.min() >= 8 and lens.max() <= 32
        assert np.all(m.values > 0)


def test_zipf_poisson_shape():
    q, i, _ = synth.make_workload("mid", n_item=30000)
    _canonical(i)
    lens = np.diff(i.indptr)
    assert lens.min() >= 1 and abs(lens.mean() - 43) < 0.5
    # heaviest rank is dim 0; it sits in nearly every row (Zipf 1.1, ~43 distinct draws)
    df = np.bincount(i.indices, minlength=i.n_cols) / i.n_rows
    assert df[0] > 0.99 and df[0] >= df[1] >= df[2] >= df[10]
    assert np.all(i.values > 0)


def test_dense_and_edge_shapes():
    q, i, _ = synth.make_workload("dense", n_item=5000, n_query=100)
    _canonical(i)
    lens = np.diff(i.indptr)
    assert abs(lens.mean() - 120) < 2
    assert np.all(i.values > 0)
    q, i, ex = synth.make_workload("edge", n_item=20000, n_query=300)
    _canonical(i)
    lens = np.diff(i.indptr)
    assert lens.max() <= 2000 and (lens == 0).mean() >= 0.01
    assert (i.values < 0).any() and (i.values > 0).any()
    perm = ex["query_item"]
    assert len(np.unique(perm)) == 300
    for j in (0, 17, 299):
        qd, qv = q.row(j)
        idd, iv = i.row(int(perm[j]))
        assert np.array_equal(qd, idd) and np.array_equal(qv, iv)
