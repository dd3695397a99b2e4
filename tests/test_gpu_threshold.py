"""Threshold-filtered output (every score >= t as a (row, item, score) hit),
for the threshold filtering the page's downstream logic applies to the full
matrix (§2.3 of "稀疏嵌入批量相似度计算的工程化实践"), through the C ABI.

The decision S >= t is taken in float32 on the exact path's scores, so the
kept set must equal {(q, j) : dense fp32 output >= t} bit for bit, with the
same scores. Against the float64 oracle, every pair farther than the score
bar (1e-5) from t is classified as the oracle's score says.
"""
import os
import sys

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

TOL = 1e-5


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


def _prepared(env, q, items, chunk):
    torch, sps, dev = env
    it = sps.prepare(sps.CSR.from_host(items, dev), chunk_size=chunk)
    qq = sps.prepare_queries(sps.CSR.from_host(q, dev), it)
    return it, qq


def _dense_and_hits(env, it, qq, n_q, t, capacity, chunks=None):
    """Exact dense scores (float32, n_q x n_items of the chunks) and the hits of
    the same chunks appended into one buffer."""
    torch, sps, dev = env
    chunks = range(it.num_chunks) if chunks is None else chunks
    width = min(it.chunk_size, it.n_items)
    out = torch.empty(n_q, width, dtype=torch.float32, device=dev)
    rs_d = torch.empty(n_q, dtype=torch.float64, device=dev)
    rs_t = torch.empty(n_q, dtype=torch.float64, device=dev)
    hits = torch.zeros(max(capacity, 0), 3, dtype=torch.int32, device=dev)
    count = torch.zeros(1, dtype=torch.int64, device=dev)
    dense = {}
    for c in chunks:
        sps.cosine_chunk(qq, it, c, out, rs_d)
        sps.cosine_chunk_threshold(qq, it, c, t, hits, count, rs_t)
        n = it.chunk_len(c)
        dense[c] = out[:, :n].cpu().numpy()
        # row sums: all of the chunk's scores, kept or not
        assert torch.allclose(rs_t, rs_d, rtol=0, atol=1e-9)
    return dense, hits, int(count.item())


def _expected(dense, chunk_size, t):
    rows, items, vals = [], [], []
    for c, d in dense.items():
        r, j = np.nonzero(d >= np.float32(t))
        rows.append(r)
        items.append(j + c * chunk_size)
        vals.append(d[r, j])
    return np.concatenate(rows), np.concatenate(items), np.concatenate(vals)


def _as_sorted(rows, items, vals):
    key = rows.astype(np.int64) * (1 << 32) + items.astype(np.int64)
    o = np.argsort(key)
    return key[o], vals[o]


def test_threshold_mid_vs_dense_and_oracle(env, orc):
    torch, sps, dev = env
    q, items, _ = synth.make_workload("mid")
    it, qq = _prepared(env, q, items, 8192)
    t = 0.3
    _, _, need = _dense_and_hits(env, it, qq, q.n_rows, t, 0)  # counting pass
    dense, hits, count = _dense_and_hits(env, it, qq, q.n_rows, t, need)
    er, ei, ev = _expected(dense, 8192, t)
    assert count == need == len(er) and count > 0
    gr, gi, gv = sps.hits_to_numpy(hits, count)
    ek, evs = _as_sorted(er, ei, ev)
    gk, gvs = _as_sorted(gr, gi, gv)
    assert np.array_equal(ek, gk)
    assert np.array_equal(evs.view(np.uint32), gvs.view(np.uint32))
    # against the oracle: pairs clear of the threshold by the score bar
    ref = orc.scores(q, items)
    kept = np.zeros(ref.shape, dtype=bool)
    kept[gr, gi] = True
    sure_in = ref >= t + TOL
    sure_out = ref < t - TOL
    assert np.all(kept[sure_in]) and not np.any(kept[sure_out])
    report("threshold %.2f mid 2000x100000: %d hits = dense >= t, oracle-consistent "
           "(%d within 1e-5 of t)" % (t, count, int((~sure_in & ~sure_out).sum())))


def test_threshold_keep_all_and_overflow(env):
    torch, sps, dev = env
    q, items, _ = synth.make_workload("tiny")
    it, qq = _prepared(env, q, items, 1000)
    # t below every score: every score of the matrix is a hit
    dense, hits, count = _dense_and_hits(env, it, qq, q.n_rows, -2.0, q.n_rows * items.n_rows)
    assert count == q.n_rows * items.n_rows
    ek, evs = _as_sorted(*_expected(dense, 1000, -2.0))
    gk, gvs = _as_sorted(*sps.hits_to_numpy(hits, count))
    assert np.array_equal(ek, gk) and np.array_equal(evs.view(np.uint32), gvs.view(np.uint32))
    # slices whose length is not a multiple of 4 (1001; 1024 and 1023): a lane's last group of
    # four scores is partial, and every score of it must still be kept
    for chunk in (1001, 2047):
        it2, qq2 = _prepared(env, q, items, chunk)
        dense, hits, count = _dense_and_hits(env, it2, qq2, q.n_rows, -2.0,
                                             q.n_rows * items.n_rows)
        assert count == q.n_rows * items.n_rows, chunk
        ek, evs = _as_sorted(*_expected(dense, chunk, -2.0))
        gk, gvs = _as_sorted(*sps.hits_to_numpy(hits, count))
        assert np.array_equal(ek, gk) and np.array_equal(evs.view(np.uint32), gvs.view(np.uint32))
    # capacity smaller than the hits: all counted, the first `capacity` written and valid
    t = 0.1
    dense, hits, count = _dense_and_hits(env, it, qq, q.n_rows, t, 0)
    full = count
    assert full > 100
    cap = full // 3
    dense, hits, count = _dense_and_hits(env, it, qq, q.n_rows, t, cap)
    assert count == full
    gr, gi, gv = sps.hits_to_numpy(hits, count)
    assert len(gr) == cap
    d = np.concatenate([dense[c] for c in sorted(dense)], axis=1)
    assert np.array_equal(d[gr, gi].view(np.uint32), gv.view(np.uint32)) and np.all(gv >= t)
    assert len(set(zip(gr.tolist(), gi.tolist()))) == cap
    report("threshold tiny: keep-all (%d hits; slices of 1000, 1001, 1024 + 1023 items) and "
           "capacity %d of %d" % (q.n_rows * items.n_rows, cap, full))


def test_threshold_pages_full_size(env):
    """Full pages shape, 3 chunks in the benchmark's launch configuration: the
    kept set equals the dense output >= t."""
    torch, sps, dev = env
    q, items, _ = synth.make_workload("pages")
    it, qq = _prepared(env, q, items, 8192)
    t = 0.3
    chunks = [0, it.num_chunks // 2, it.num_chunks - 1]
    # a counting pass (capacity 0) sizes the hit buffer
    _, _, need = _dense_and_hits(env, it, qq, q.n_rows, t, 0, chunks)
    dense, hits, count = _dense_and_hits(env, it, qq, q.n_rows, t, need, chunks)
    assert count == need
    ek, evs = _as_sorted(*_expected(dense, 8192, t))
    gk, gvs = _as_sorted(*sps.hits_to_numpy(hits, count))
    assert count == len(ek) and np.array_equal(ek, gk)
    assert np.array_equal(evs.view(np.uint32), gvs.view(np.uint32))
    report("threshold %.2f pages, 3 chunks: %d hits = dense >= t" % (t, count))


def test_threshold_arguments(env):
    torch, sps, dev = env
    q, items, _ = synth.make_workload("tiny", n_item=100, n_query=5)
    it, qq = _prepared(env, q, items, 64)
    hits = torch.zeros(10, 3, dtype=torch.int32, device=dev)
    count = torch.zeros(1, dtype=torch.int64, device=dev)
    with pytest.raises(sps.SpsError):
        sps.cosine_chunk_threshold(qq, it, it.num_chunks, 0.5, hits, count)
    with pytest.raises(sps.SpsError):
        sps.cosine_chunk_threshold(qq, it, 0, float("nan"), hits, count)


def test_threshold_ragged_groups_and_dense_off(env, orc, monkeypatch):
    """300 queries (the last 16-row group holds 12), 2048-item chunks (two slices
    per chunk, partial row sums folded), the heavy-dim part on and off."""
    torch, sps, dev = env
    q, items, extra = synth.make_workload("edge", n_item=6000, n_query=300)
    ref = orc.scores(q, items)
    for dense_on in ("1", "0"):
        monkeypatch.setenv("SPS_DENSE", dense_on)
        it, qq = _prepared(env, q, items, 2048)
        t = 0.2
        _, _, need = _dense_and_hits(env, it, qq, q.n_rows, t, 0)
        dense, hits, count = _dense_and_hits(env, it, qq, q.n_rows, t, need)
        ek, evs = _as_sorted(*_expected(dense, 2048, t))
        gr, gi, gv = sps.hits_to_numpy(hits, count)
        gk, gvs = _as_sorted(gr, gi, gv)
        assert count == need == len(ek) and np.array_equal(ek, gk)
        assert np.array_equal(evs.view(np.uint32), gvs.view(np.uint32))
        assert np.any(gr >= 288)  # the ragged group contributes
        kept = np.zeros(ref.shape, dtype=bool)
        kept[gr, gi] = True
        assert np.all(kept[ref >= t + TOL]) and not np.any(kept[ref < t - TOL])
        report("threshold %.2f edge 300x6000, chunk 2048, dense=%s: %d hits = dense >= t, "
               "oracle-consistent" % (t, dense_on, count))
