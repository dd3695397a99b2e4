"""The reduced-precision variant (fp16 item values, fp16 scores) against the
float64 oracle, through the C ABI.

The page allows fp16 value data where a loss below 1e-3 is acceptable, with
the norms kept in float32 (§5.3 of "稀疏嵌入批量相似度计算的工程化实践"). The
bar is that bound for every score: the item values contribute at most 2^-11
and the fp16 output rounding at most 2^-11 (include/sps.h derives both), so
|S_half - S| < 1e-3. The exact path is the oracle here too.
"""
import os
import sys

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

HALF_TOL = 1e-3


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_embedding_exact_amd as sps
    sps.load_library()
    return torch, sps, torch.device("cuda:0")


def report(name, err, n, bar=HALF_TOL):
    line = "[parity] %-44s n=%-11d max|err|=%.3g (bar %.3g; fp16 variant)" % (name, n, err, bar)
    print("\n" + line, file=sys.stderr, flush=True)
    path = os.environ.get("SPS_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(line + "\n")


def half_chunks(env, q, items, chunk_size, rows=None):
    """Yield (begin, fp16 scores as float64 [rows or all, chunk_len], row sums)."""
    torch, sps, dev = env
    it = sps.prepare(sps.CSR.from_host(items, dev), chunk_size=chunk_size)
    it.enable_half()
    qq = sps.prepare_queries(sps.CSR.from_host(q, dev), it)
    width = min(chunk_size, items.n_rows)
    out = torch.empty(q.n_rows, width, dtype=torch.float16, device=dev)
    rs = torch.empty(q.n_rows, dtype=torch.float64, device=dev)
    sel = None if rows is None else torch.as_tensor(np.asarray(rows), device=dev)
    for c in range(it.num_chunks):
        sps.cosine_chunk_half(qq, it, c, out, rs)
        n = it.chunk_len(c)
        full = out[:, :n].double()
        # the checksum is the float64 sum of the fp16 values written
        assert torch.allclose(rs, full.sum(1), rtol=0, atol=1e-9)
        o = full if sel is None else full[sel]
        yield c * chunk_size, o.cpu().numpy()


def test_half_tiny_and_mid_all_scores(env, orc):
    for name, chunk in (("tiny", 4096), ("mid", 8192)):
        q, items, _ = synth.make_workload(name)
        qn, _ = orc.row_norms(q)
        inn, _ = orc.row_norms(items)
        worst, n = 0.0, 0
        for b, got in half_chunks(env, q, items, chunk):
            ref = orc.scores(q, items, q_norm=qn, i_norm=inn, item_begin=b,
                             item_end=b + got.shape[1])
            worst = max(worst, float(np.abs(got - ref).max()))
            n += got.size
        report("half %s all scores" % name, worst, n)
        assert n == q.n_rows * items.n_rows
        assert worst < HALF_TOL


@pytest.mark.parametrize("name,n_rows", [("pages", 32), ("dense", 64)])
def test_half_sampled_rows(env, orc, name, n_rows):
    w = synth.WORKLOADS[name]
    q, items, _ = synth.make_workload(name)
    rows = np.sort(np.random.default_rng(99).choice(q.n_rows, n_rows, replace=False))
    got = np.concatenate([g for _, g in half_chunks(env, q, items, w.chunk_size, rows)], axis=1)
    ref = orc.scores(q, items, q_rows=rows)
    err = float(np.abs(got - ref).max())
    report("half %s %d sampled rows x all items" % (name, n_rows), err, got.size)
    assert err < HALF_TOL


def test_half_self_scores_and_dense_off(env, orc, monkeypatch):
    """Identical rows (S = 1, the worst case of the output rounding) and the
    inverted-list-only kernel (SPS_DENSE=0)."""
    torch, sps, dev = env
    for dense in ("1", "0"):
        monkeypatch.setenv("SPS_DENSE", dense)
        q, items, extra = synth.make_workload("edge", n_item=6000, n_query=300)
        perm = extra["query_item"]
        ref = orc.scores(q, items)
        got = np.concatenate([g for _, g in half_chunks(env, q, items, 2048)], axis=1)
        err = float(np.abs(got - ref).max())
        inside = perm < items.n_rows
        nonempty = np.diff(q.indptr) > 0
        sel = np.nonzero(inside & nonempty)[0]
        self_err = float(np.abs(got[sel, perm[sel]] - 1.0).max())
        report("half edge 300x6000 dense=%s (self %d)" % (dense, len(sel)), err, got.size)
        assert err < HALF_TOL and self_err < HALF_TOL


def test_half_reproducible_and_close_to_exact_path(env):
    """Two runs are bitwise equal, and at the full pages size (a few chunks)
    every fp16 score is within the bound of the exact path's fp32 score
    (which is within 1e-5 of the oracle)."""
    torch, sps, dev = env
    q, items, _ = synth.make_workload("pages")
    it = sps.prepare(sps.CSR.from_host(items, dev), chunk_size=8192)
    it.enable_half()
    qq = sps.prepare_queries(sps.CSR.from_host(q, dev), it)
    o16 = torch.empty(q.n_rows, 8192, dtype=torch.float16, device=dev)
    o16b = torch.empty_like(o16)
    o32 = torch.empty(q.n_rows, 8192, dtype=torch.float32, device=dev)
    worst = 0.0
    for c in (0, it.num_chunks // 2, it.num_chunks - 1):
        n = it.chunk_len(c)
        sps.cosine_chunk_half(qq, it, c, o16)
        sps.cosine_chunk_half(qq, it, c, o16b)
        sps.cosine_chunk(qq, it, c, o32)
        assert torch.equal(o16[:, :n], o16b[:, :n])
        worst = max(worst, float((o16[:, :n].float() - o32[:, :n]).abs().max()))
    report("half vs exact path, pages, 3 chunks", worst, 3 * q.n_rows * 8192)
    assert worst < HALF_TOL - 1e-5


def test_half_needs_enable(env):
    torch, sps, dev = env
    q, items, _ = synth.make_workload("tiny", n_item=100, n_query=5)
    it = sps.prepare(sps.CSR.from_host(items, dev), chunk_size=64)
    qq = sps.prepare_queries(sps.CSR.from_host(q, dev), it)
    out = torch.empty(5, 64, dtype=torch.float16, device=dev)
    with pytest.raises(sps.SpsError):
        sps.cosine_chunk_half(qq, it, 0, out)
    it.enable_half()
    sps.cosine_chunk_half(qq, it, 0, out)
    with pytest.raises(sps.SpsError):
        sps.cosine_chunk_half(qq, it, it.num_chunks, out)
