"""GPU path vs the float64 oracle, through the C ABI.

Bars: bit-exact for index structures (inverted lists) and for the fp32
inverse norms (both sides round fl32(1/sqrt(float64 sum)) once); max
|S_gpu - S_oracle| <= 1e-5 for scores (the achieved maximum is printed
against the page's 1e-6 goal, §2.3 of "稀疏嵌入批量相似度计算的工程化实践").
"""
import os
import sys

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

TOL = 1e-5
SLICE_MAX = 1024  # items per slice at most (the prepare call's slice rule)

# Per-score rounding budget of the GPU path (derived in the design notes, §4):
#   |S_gpu - S| <= EPS_ABS * A + EPS_TERM * (m + b)
# with A = sum_d |q^_d i^_d| over the shared dims, m their number, b the
# heavy-dim blocks (1 to 4; 1 when there are none), u = 2^-24: inputs rounded
# once to fp32 (2u), fp32 products (u), the heavy dims' split fp16 (3 * 2^-22
# = 12u) and fp32 accumulation within a block of 32 dims (< 32u of the
# block's part of A), the final fp32 conversion (u |S| <= u A): below 49u of A
# in all; every light product and each block's dense sum are rounded once to
# 2^-30 fixed point (2^-31 each).
# Sums of scores add the per-score bounds, whose sums over a chunk row or an
# item column are closed forms of the oracle (kinds 1 and 2); float64 summation
# adds far less than FP64_SLACK.
EPS_ABS = 49.0 * 2.0 ** -24
EPS_TERM = 2.0 ** -31
FP64_SLACK = 1e-7


def sum_bar(abs_sums, counts, n_terms, blocks=1):
    """Bound on |sum of GPU scores - sum of exact scores| over n_terms pairs
    (blocks: the corpus's heavy-dim blocks)."""
    return EPS_ABS * abs_sums + EPS_TERM * (counts + max(1, blocks) * n_terms) + FP64_SLACK


def heavy_blocks(it):
    return (len(it.heavy_dims()) + 31) // 32


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_embedding_exact_amd as sps
    sps.load_library()
    return torch, sps, torch.device("cuda:0")


def report(name, err, n, bar=TOL):
    line = "[parity] %-44s n=%-11d max|err|=%.3g (bar %.3g; page goal 1e-6 per score)" % (
        name, n, err, bar)
    print("\n" + line, file=sys.stderr, flush=True)
    path = os.environ.get("SPS_PARITY_LOG")
    if path:
        with open(path, "a") as f:
            f.write(line + "\n")


def gpu_chunks(env, q, items, chunk_size, rows=None, sums=False):
    """Yield (c, begin, scores[rows or all, chunk_len] numpy, row_sums numpy|None)."""
    torch, sps, dev = env
    it = sps.prepare(sps.CSR.from_host(items, dev), chunk_size=chunk_size)
    qq = sps.prepare_queries(sps.CSR.from_host(q, dev), it)
    width = min(chunk_size, items.n_rows)
    out = torch.empty(q.n_rows, width, dtype=torch.float32, device=dev)
    rs = torch.empty(q.n_rows, dtype=torch.float64, device=dev) if sums else None
    sel = None if rows is None else torch.as_tensor(np.asarray(rows), device=dev)
    for c in range(it.num_chunks):
        sps.cosine_chunk(qq, it, c, out, rs)
        n = it.chunk_len(c)
        o = out[:, :n] if sel is None else out[sel, :n]
        yield c, c * chunk_size, o.cpu().numpy(), (rs.cpu().numpy() if sums else None)


# ---------------------------------------------------------------------------
# norms and inverted lists: bit-exact
# ---------------------------------------------------------------------------

def _check_structures(env, orc, items, chunk_size, name, slices=None):
    torch, sps, dev = env
    n64, inv32 = orc.row_norms(items)
    it = sps.prepare(sps.CSR.from_host(items, dev), chunk_size=chunk_size)
    assert it.slices_per_chunk == -(-chunk_size // SLICE_MAX)
    for sl in (range(it.num_slices) if slices is None else slices(it)):
        v = it.slice_view(sl)
        b = v["item_begin"]
        e = b + v["slice_len"]
        col_ptr, row, val = orc.chunk_csc(items, n64, b, e)
        assert v["slice_nnz"] == len(row), (name, sl)
        g_cp, consistent = it.slice_col_ptr(sl)
        assert consistent, (name, sl, "dim index lengths")
        assert np.array_equal(g_cp.cpu().numpy(), col_ptr), (name, sl, "col_ptr")
        post = v["post"].cpu().numpy()
        g_row = post[:, 0]
        assert np.array_equal(g_row, row), (name, sl, "row ids")
        g_val = post[:, 1].copy().view(np.float32)
        assert np.array_equal(g_val.view(np.uint32), val.view(np.uint32)), (name, sl, "values")
        g_inv = v["item_inv_norm"].cpu().numpy()
        assert np.array_equal(g_inv.view(np.uint32), inv32[b:e].view(np.uint32)), (name, sl)
    if slices is None:
        # the slices tile every chunk in order
        ends = [it.slice_view(sl)["item_begin"] + it.slice_view(sl)["slice_len"]
                for sl in range(it.num_slices)]
        assert max(ends) == items.n_rows
    n_checked = it.num_slices if slices is None else len(list(slices(it)))
    print("\n[parity] %s: %d slices, inverted lists + norms bit-exact" % (name, n_checked),
          file=sys.stderr, flush=True)
    return it


def test_structures_tiny(env, orc):
    _, items, _ = synth.make_workload("tiny")
    _check_structures(env, orc, items, 4096, "tiny")


def test_structures_zipf_ragged(env, orc):
    _, items, _ = synth.make_workload("mid", n_item=30001)
    _check_structures(env, orc, items, 8192, "mid 30001 items (ragged tail)")


def test_structures_dense_and_edge(env, orc):
    _, items, _ = synth.make_workload("dense", n_item=20000)
    _check_structures(env, orc, items, 8192, "dense 20000 items")
    _, items, _ = synth.make_workload("edge", n_item=17000)
    _check_structures(env, orc, items, 8192, "edge 17000 items (empty rows, signed)")


@pytest.mark.parametrize("cap", ["0", "1"])
def test_structures_dim_index_fallback(env, orc, cap, monkeypatch):
    """The dim index built with room for fewer deferred runs than the slices
    defer (SPS_DIM_DEFER_CAP; runs whose probe leaves an LDS range of the
    table are deferred): the rest go in through the fallback sweep, and the
    index must come out the same."""
    monkeypatch.setenv("SPS_DIM_DEFER_CAP", cap)
    _, items, _ = synth.make_workload("mid", n_item=30001)
    _check_structures(env, orc, items, 8192, "mid 30001 items, deferred-run cap %s" % cap)
    _, items, _ = synth.make_workload("edge", n_item=17000)
    _check_structures(env, orc, items, 8192, "edge 17000 items, deferred-run cap %s" % cap)


@pytest.mark.parametrize("name", ["pages", "dense", "edge"])
def test_structures_full_size_sample(env, orc, name):
    """Bit-exact inverted lists on a seeded sample of the full-size corpora's
    slices: the first and last slice, every slice of the last (partial) chunk,
    and 16 random others."""
    w = synth.WORKLOADS[name]
    _, items, _ = synth.make_workload(name)

    def pick(it):
        spc = it.slices_per_chunk
        rng = np.random.default_rng(4321)
        chosen = {0, it.num_slices - 1}
        chosen |= set(range((it.num_chunks - 1) * spc, it.num_slices))
        chosen |= set(rng.choice(it.num_slices, 16, replace=False).tolist())
        return sorted(chosen)
    _check_structures(env, orc, items, w.chunk_size, "%s full size, sampled slices" % name,
                      slices=pick)


def test_query_inverse_norms(env, orc):
    torch, sps, dev = env
    for name, kw in [("tiny", {}), ("edge", {"n_item": 5000, "n_query": 777})]:
        q, items, _ = synth.make_workload(name, **kw)
        _, inv32 = orc.row_norms(q)
        got = sps.row_inv_norms(sps.CSR.from_host(q, dev)).cpu().numpy()
        assert np.array_equal(got.view(np.uint32), inv32.view(np.uint32)), name
        it = sps.prepare(sps.CSR.from_host(items, dev), chunk_size=4096)
        qq = sps.prepare_queries(sps.CSR.from_host(q, dev), it)
        assert np.array_equal(qq.inv_norm.cpu().numpy().view(np.uint32), inv32.view(np.uint32))


# ---------------------------------------------------------------------------
# scores: every score on the two small workloads
# ---------------------------------------------------------------------------

def test_scores_tiny_full(env, orc):
    q, items, _ = synth.make_workload("tiny")
    ref = orc.scores(q, items)
    (c, b, got, _), = list(gpu_chunks(env, q, items, 4096))
    err = float(np.abs(got - ref).max())
    report("tiny 256x4096 all scores", err, got.size)
    assert err <= TOL


def test_scores_mid_full(env, orc):
    q, items, _ = synth.make_workload("mid")
    worst, n = 0.0, 0
    qn, _ = orc.row_norms(q)
    inn, _ = orc.row_norms(items)
    for c, b, got, rs in gpu_chunks(env, q, items, 8192, sums=True):
        ref = orc.scores(q, items, q_norm=qn, i_norm=inn, item_begin=b,
                         item_end=b + got.shape[1])
        worst = max(worst, float(np.abs(got - ref).max()))
        n += got.size
        assert np.abs(rs - got.astype(np.float64).sum(1)).max() <= 1e-9
    report("mid 2000x100000 all scores (13 chunks)", worst, n)
    assert n == 2000 * 100000
    assert worst <= TOL


# ---------------------------------------------------------------------------
# full-size workloads: sampled rows x all items + closed-form row sums of
# every chunk (the sums of the exact scores, by linearity)
# ---------------------------------------------------------------------------

def _sampled(env, orc, name, n_rows_sampled, self_scores=False, col_chunks=()):
    w = synth.WORKLOADS[name]
    q, items, extra = synth.make_workload(name)
    rng = np.random.default_rng(1234)
    rows = np.sort(rng.choice(q.n_rows, n_rows_sampled, replace=False))
    qn, _ = orc.row_norms(q)
    inn, _ = orc.row_norms(items)
    ref_sums = orc.chunk_row_sums(q, items, w.chunk_size, q_norm=qn, i_norm=inn)
    abs_sums = orc.chunk_row_sums(q, items, w.chunk_size, q_norm=qn, i_norm=inn, kind=1)
    cnt_sums = orc.chunk_row_sums(q, items, w.chunk_size, q_norm=qn, i_norm=inn, kind=2)
    max_abs = 0.0  # largest |S| over the whole matrix
    col_worst = 0.0  # largest column-sum error / its bar
    worst, worst_sum, n = 0.0, 0.0, 0
    self_err = 0.0
    torch, sps, dev = env
    it = sps.prepare(sps.CSR.from_host(items, dev), chunk_size=w.chunk_size)
    qq = sps.prepare_queries(sps.CSR.from_host(q, dev), it)
    nblk = heavy_blocks(it)
    out = torch.empty(q.n_rows, w.chunk_size, dtype=torch.float32, device=dev)
    rs = torch.empty(it.num_chunks, q.n_rows, dtype=torch.float64, device=dev)
    sel = torch.as_tensor(rows, device=dev)
    got_rows = np.empty((len(rows), items.n_rows), dtype=np.float32)
    self_cols = None
    if self_scores:
        perm = extra["query_item"]
        self_vals = np.full(q.n_rows, np.nan, dtype=np.float64)
    for c in range(it.num_chunks):
        sps.cosine_chunk(qq, it, c, out, rs[c])
        n_c = it.chunk_len(c)
        b = c * w.chunk_size
        got_rows[:, b:b + n_c] = out[sel, :n_c].cpu().numpy()
        max_abs = max(max_abs, float(out[:, :n_c].abs().max().item()))
        if c in col_chunks:
            g_col = out[:, :n_c].double().sum(0).cpu().numpy()
            r_col = orc.col_sums(q, items, b, b + n_c, q_norm=qn, i_norm=inn)
            bar = sum_bar(orc.col_sums(q, items, b, b + n_c, q_norm=qn, i_norm=inn, kind=1),
                          orc.col_sums(q, items, b, b + n_c, q_norm=qn, i_norm=inn, kind=2),
                          q.n_rows, nblk)
            e_col = np.abs(g_col - r_col)
            report("%s column sums, chunk %d (%d items); worst err/bar %.3f" % (
                name, c, n_c, float((e_col / bar).max())), float(e_col.max()), n_c,
                bar=float(bar[np.argmax(e_col)]))
            assert np.all(e_col <= bar), (c, int(np.argmax(e_col - bar)))
            col_worst = max(col_worst, float((e_col / bar).max()))
        if self_scores:
            inside = np.nonzero((perm >= b) & (perm < b + n_c))[0]
            if len(inside):
                qi = torch.as_tensor(inside, device=dev)
                cj = torch.as_tensor(perm[inside] - b, device=dev)
                self_vals[inside] = out[qi, cj].double().cpu().numpy()
    torch.cuda.synchronize()
    ref = orc.scores(q, items, q_norm=qn, i_norm=inn, q_rows=rows)
    worst = float(np.abs(got_rows - ref).max())
    n = got_rows.size
    g_sums = rs.cpu().numpy()
    e_sums = np.abs(g_sums - ref_sums)
    worst_sum = float(e_sums.max())
    chunk_lens = np.array([it.chunk_len(c) for c in range(it.num_chunks)], dtype=np.float64)
    bars = sum_bar(abs_sums, cnt_sums, chunk_lens[:, None], nblk)
    report("%s %d sampled rows x all items" % (name, len(rows)), worst, n)
    err_all = np.abs(got_rows - ref)
    within = float((err_all <= 1e-6).mean())
    report("%s share of compared scores within 1e-6: %.6f" % (name, within), worst, n, bar=1e-6)
    report("%s max |S| over all %d scores: excess over 1 = %.3g" % (
        name, q.n_rows * items.n_rows, max(0.0, max_abs - 1.0)), max(0.0, max_abs - 1.0),
        q.n_rows * items.n_rows)
    report("%s row sums, %d chunks x %d rows; worst err/bar %.3f" % (
        name, it.num_chunks, q.n_rows, float((e_sums / bars).max())), worst_sum,
        it.num_chunks * q.n_rows, bar=float(bars.flat[np.argmax(e_sums)]))
    assert worst <= TOL
    assert max_abs <= 1.0 + TOL  # no clamp; |S| <= 1 up to rounding
    assert np.all(e_sums <= bars), np.unravel_index(int(np.argmax(e_sums - bars)), bars.shape)
    if self_scores:
        empty = np.diff(q.indptr) == 0
        self_err = float(np.abs(self_vals[~empty] - 1.0).max())
        report("%s self-scores (%d empty rows -> 0)" % (name, int(empty.sum())), self_err,
               int((~empty).sum()))
        assert self_err <= TOL
        assert np.all(self_vals[empty] == 0.0)


def test_pages_shape_sampled(env, orc):
    _sampled(env, orc, "pages", 64, col_chunks=(0, 122, 244))


def test_dense_overlap_sampled(env, orc):
    _sampled(env, orc, "dense", 128, col_chunks=(0, 61))


def test_edge_heavy_tail_sampled(env, orc):
    _sampled(env, orc, "edge", 128, self_scores=True, col_chunks=(0, 122))


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------

def _dense_ref(orc, q, items):
    return orc.scores(q, items)


@pytest.mark.parametrize("dense", ["1", "0"])
def test_dense_rows_on_and_off(env, orc, dense, monkeypatch):
    """Heavy dims through the matrix-core rows (default) or all through the
    inverted lists (SPS_DENSE=0); odd query count (not a multiple of 16)."""
    monkeypatch.setenv("SPS_DENSE", dense)
    torch, sps, dev = env
    q, items, _ = synth.make_workload("mid", n_item=9001, n_query=37)
    it = sps.prepare(sps.CSR.from_host(items, dev), chunk_size=4096)
    heavy = it.heavy_dims()
    if dense == "1":
        # Zipf(1.1): the lowest dims are in most rows; the choice is the most frequent dims
        df = np.bincount(items.indices, minlength=items.n_cols)
        top = set(np.argsort(-df, kind="stable")[:len(heavy)].tolist())
        assert 16 <= len(heavy) <= 32 and heavy == sorted(heavy) and set(heavy) <= top | set(heavy)
        assert all(df[h] >= items.n_rows / 16 for h in heavy)
    else:
        assert heavy == []
    ref = orc.scores(q, items)
    got = np.concatenate([g for _, _, g, _ in gpu_chunks(env, q, items, 4096)], axis=1)
    err = float(np.abs(got - ref).max())
    report("dense=%s 37x9001 chunk 4096" % dense, err, got.size)
    assert err <= TOL


def expected_heavy(items, chunk_size, cap=128, gain=0.4):
    """The heavy-dim rule, restated on the host. A dim's frequency counts the
    items of each slice whose list of that dim holds at least 1/32 of the
    slice size (so that dims held here and there do not qualify); candidates
    reach 1/16 of the items; ranked by that frequency (ties to the lower dim):
    the first block of 32, and block b while the sum over its dims of
    (df / n)^2 exceeds `gain`; at most `cap` dims."""
    n = items.n_rows
    n_sub = -(-chunk_size // SLICE_MAX)
    S = -(-chunk_size // n_sub)
    hmin = max(2, S // 32)
    df = np.zeros(items.n_cols, dtype=np.int64)
    for c0 in range(0, n, chunk_size):
        c1 = min(n, c0 + chunk_size)
        for s0 in range(c0, c1, S):
            s1 = min(c1, s0 + S)
            cnt = np.bincount(items.indices[items.indptr[s0]:items.indptr[s1]],
                              minlength=items.n_cols)
            df += np.where(cnt >= hmin, cnt, 0)
    t = max(2, -(-n // 16))
    cand = np.nonzero(df >= t)[0]
    order = cand[np.lexsort((cand, -df[cand]))]
    lim = min(len(order), cap)
    top = df[order[:lim]].astype(np.float64)
    nb = 1
    while nb < -(-lim // 32) and float((top[32 * nb:32 * nb + 32] ** 2).sum()) > gain * float(n) ** 2:
        nb += 1
    return sorted(order[:min(lim, 32 * nb)].tolist()) if lim > 0 else []


def test_heavy_choice_is_deterministic(env):
    """Dense-overlap items (Zipf 1.0 over 30,522 dims): four blocks of 32
    heavy dims, the ones the rule picks, the same on every prepare."""
    torch, sps, dev = env
    _, items, _ = synth.make_workload("dense", n_item=30000)
    a = sps.prepare(sps.CSR.from_host(items, dev), chunk_size=8192).heavy_dims()
    b = sps.prepare(sps.CSR.from_host(items, dev), chunk_size=8192).heavy_dims()
    assert a == b and len(a) == 128
    assert a == expected_heavy(items, 8192)


@pytest.mark.parametrize("gain,cap", [("0", "128"), ("0", "40"), ("0.4", "128"), ("0.4", "0")])
def test_heavy_blocks(env, orc, gain, cap, monkeypatch):
    """The heavy-dim blocks: every further block forced (gain 0: as many
    blocks as the candidates fill, the last one partial), a cap of 40 (a
    second block of 8 dims), the default rule (one block on this Zipf(1.1)
    corpus) and no heavy dims at all; each the rule's choice, and every score
    within the bar of the oracle and within rounding of the path without
    the dense part."""
    monkeypatch.setenv("SPS_HEAVY_GAIN", gain)
    monkeypatch.setenv("SPS_HEAVY_MAX", cap)
    torch, sps, dev = env
    q, items, _ = synth.make_workload("mid", n_item=9001, n_query=37)
    it = sps.prepare(sps.CSR.from_host(items, dev), chunk_size=4096)
    heavy = it.heavy_dims()
    assert heavy == expected_heavy(items, 4096, int(cap), float(gain))
    if gain == "0" and cap == "128":
        assert len(heavy) > 64  # three blocks at least
    if cap == "40":
        assert len(heavy) == 40
    ref = orc.scores(q, items)
    got = np.concatenate([g for _, _, g, _ in gpu_chunks(env, q, items, 4096)], axis=1)
    err = float(np.abs(got - ref).max())
    report("heavy gain %s cap %s (%d dims) 37x9001" % (gain, cap, len(heavy)), err, got.size)
    assert err <= TOL
    monkeypatch.setenv("SPS_DENSE", "0")
    flat = np.concatenate([g for _, _, g, _ in gpu_chunks(env, q, items, 4096)], axis=1)
    assert float(np.abs(got - flat).max()) <= 2e-6


def test_bitwise_reproducible(env):
    """Integer accumulation: repeated runs give identical bits."""
    torch, sps, dev = env
    q, items, _ = synth.make_workload("mid", n_item=12000, n_query=100)
    runs = [np.concatenate([g for _, _, g, _ in gpu_chunks(env, q, items, 8192)], axis=1)
            for _ in range(3)]
    assert all(np.array_equal(runs[0].view(np.uint32), r.view(np.uint32)) for r in runs[1:])


def test_row_permutation_invariance(env):
    """A query's scores do not depend on the rows it is grouped with: the light
    sums are integers in any order (the query prepare sorts each 16-row group's
    records by dim) and the heavy part is per row. The batch scored in a
    shuffled row order, then unshuffled, is bitwise equal to the original."""
    torch, sps, dev = env
    from synth import HostCSR
    q, items, _ = synth.make_workload("mid", n_item=12000, n_query=203)
    perm = np.random.default_rng(17).permutation(q.n_rows)
    cnt = np.diff(q.indptr)[perm]
    ip = np.concatenate([[0], np.cumsum(cnt)]).astype(np.int32)
    ix = np.concatenate([q.indices[q.indptr[r]:q.indptr[r + 1]] for r in perm])
    vx = np.concatenate([q.values[q.indptr[r]:q.indptr[r + 1]] for r in perm])
    qp = HostCSR(ip, ix.astype(np.int32), vx.astype(np.float32), q.n_rows, q.n_cols)
    a = np.concatenate([g for _, _, g, _ in gpu_chunks(env, q, items, 8192)], axis=1)
    b = np.concatenate([g for _, _, g, _ in gpu_chunks(env, qp, items, 8192)], axis=1)
    assert np.array_equal(a[perm].view(np.uint32), b.view(np.uint32))
    report("mid 203x12000 rows shuffled: bitwise equal", 0.0, a.size)


def test_group_first_batch_misses_slice(env, orc):
    """One 16-row group with more than 1024 light entries (two batches; such a
    group keeps its records in row order): every entry of the first batch is a
    dim no item holds, so that batch has no segments, and the second batch's
    entries share dims with the slice. Scores must match the oracle."""
    from synth import HostCSR
    rng = np.random.default_rng(5)
    _, items, _ = synth.make_workload("mid", n_item=2048)
    dim_hi = items.n_cols  # query dims >= this are absent from every item
    D = dim_hi + 100000
    rows = []
    for r in range(15):
        d = np.sort(rng.choice(np.arange(dim_hi, D), 70, replace=False))
        rows.append(list(zip(d.tolist(), rng.lognormal(0, 1, 70).astype(np.float32).tolist())))
    present = np.unique(items.indices)
    d = np.sort(rng.choice(present, 60, replace=False))
    rows.append(list(zip(d.tolist(), rng.lognormal(0, 1, 60).astype(np.float32).tolist())))
    import pins
    q = pins.csr_from_rows(rows, D)
    items_d = HostCSR(items.indptr, items.indices, items.values, items.n_rows, D)
    assert q.nnz > 1024 + 40
    ref = orc.scores(q, items_d)
    got = np.concatenate([g for _, _, g, _ in gpu_chunks(env, q, items_d, 1024)], axis=1)
    err = float(np.abs(got - ref).max())
    report("16x2048: first batch of the group misses every slice", err, got.size)
    assert err <= TOL
    assert np.abs(got[15]).max() > 0.01  # the second batch did contribute


def test_wide_slice_index(env, orc):
    """A slice of more than 2^22 entries (1,024 items of 4,100 entries each) takes the
    dim index's wide format: one list per bucket, its start and its length in separate
    words. The index is built over two LDS ranges (8,192 dims, 16,384 buckets), and the
    inverted lists and scores must match the oracle."""
    from synth import HostCSR
    rng = np.random.default_rng(77)
    n_items, dim, per_row = 1024, 8192, 4100
    assert n_items * per_row > (1 << 22)
    indices = np.concatenate([np.sort(rng.choice(dim, per_row, replace=False))
                              for _ in range(n_items)]).astype(np.int32)
    indptr = (np.arange(n_items + 1, dtype=np.int64) * per_row).astype(np.int32)
    values = rng.lognormal(0, 1, indices.size).astype(np.float32)
    items = HostCSR(indptr, indices, values, n_items, dim)
    _check_structures(env, orc, items, 1024, "wide slice (4.2M entries)")
    qrows = []
    for r in range(20):
        d = np.sort(rng.choice(dim, 40 + 13 * r, replace=False))
        qrows.append(list(zip(d.tolist(), rng.lognormal(0, 1, d.size).astype(np.float32).tolist())))
    import pins
    q = pins.csr_from_rows(qrows, dim)
    ref = orc.scores(q, items)
    got = np.concatenate([g for _, _, g, _ in gpu_chunks(env, q, items, 1024)], axis=1)
    err = float(np.abs(got - ref).max())
    report("20x1024: one slice of 4.2M entries (wide dim index)", err, got.size)
    assert err <= TOL


def test_edge_rows_and_ld(env, orc):
    """Empty rows on both sides, explicit zeros, a dim no item has, a chunk
    length that is not a multiple of 4, ld > chunk_len (the tail untouched)."""
    import pins
    torch, sps, dev = env
    rng = np.random.default_rng(99)
    from synth import HostCSR
    items = pins.random_csr(rng, 1003, 5000, 0, 30, signed=True, empty_frac=0.1,
                            explicit_zero_frac=0.05)
    items = HostCSR(items.indptr, items.indices, items.values, items.n_rows, 5001)
    q = pins.random_csr(rng, 21, 5000, 0, 30, signed=True, empty_frac=0.2,
                        explicit_zero_frac=0.05)
    # a last query on dim 5000, which no item holds
    q = pins.csr_from_rows([list(zip(*q.row(r))) for r in range(q.n_rows)] + [[(5000, 1.0)]],
                           5001)
    ref = orc.scores(q, items)
    it = sps.prepare(sps.CSR.from_host(items, dev), chunk_size=333)
    qq = sps.prepare_queries(sps.CSR.from_host(q, dev), it)
    ld = 341  # not a multiple of 4: scalar stores
    big = torch.full((q.n_rows, ld), float("nan"), dtype=torch.float32, device=dev)
    worst = 0.0
    for c in range(it.num_chunks):
        big.fill_(float("nan"))
        sps.cosine_chunk(qq, it, c, big)
        n = it.chunk_len(c)
        g = big.cpu().numpy()
        assert np.isnan(g[:, n:]).all(), "columns beyond the chunk were written"
        worst = max(worst, float(np.abs(g[:, :n] - ref[:, c * 333:c * 333 + n]).max()))
    report("random signed 22x1003 chunk 333 ld 341", worst, ref.size)
    assert worst <= TOL
    # empty query rows and zero-norm items give exactly 0
    got = np.concatenate([g for _, _, g, _ in gpu_chunks(env, q, items, 333)], axis=1)
    qn, _ = orc.row_norms(q)
    inn, _ = orc.row_norms(items)
    assert np.all(got[qn == 0, :] == 0.0) and np.all(got[:, inn == 0] == 0.0)
    assert np.all(got[-1] == 0.0)


def test_chunk_size_extremes(env, orc):
    q, items, _ = synth.make_workload("tiny", n_item=1500, n_query=50)
    ref = orc.scores(q, items)
    for cs in (1, 7, 1500, 32768):
        got = np.concatenate([g for _, _, g, _ in gpu_chunks(env, q, items, cs)], axis=1)
        err = float(np.abs(got - ref).max())
        report("tiny 50x1500 chunk %d" % cs, err, got.size)
        assert err <= TOL
    # chunks cut into uneven slices (ceil(C/1024) slices, last one shorter)
    q, items, _ = synth.make_workload("mid", n_item=9001, n_query=21)
    ref = orc.scores(q, items)
    for cs in (2049, 3000, 4097, 6000):
        _check_structures(env, orc, items, cs, "mid 9001 chunk %d" % cs)
        got = np.concatenate([g for _, _, g, _ in gpu_chunks(env, q, items, cs)], axis=1)
        err = float(np.abs(got - ref).max())
        report("mid 21x9001 chunk %d" % cs, err, got.size)
        assert err <= TOL


def test_chunk_size_invariance(env):
    """Scores with 4096-item and 8192-item chunks are bitwise equal: both cut the
    items into the same 1024-item slices, pick the same heavy dims, and the
    light sums are integers."""
    q, items, _ = synth.make_workload("mid", n_item=16384, n_query=200)
    a = np.concatenate([g for _, _, g, _ in gpu_chunks(env, q, items, 4096)], axis=1)
    b = np.concatenate([g for _, _, g, _ in gpu_chunks(env, q, items, 8192)], axis=1)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_stream_entry_and_bulk(env, orc):
    torch, sps, dev = env
    q, items, _ = synth.make_workload("mid", n_item=20000, n_query=64)
    ref = orc.scores(q, items)
    full = sps.bulk_similarity(sps.CSR.from_host(q, dev), sps.CSR.from_host(items, dev),
                               chunk_size=8192)
    assert float(np.abs(full.cpu().numpy() - ref).max()) <= TOL
    it = sps.prepare(sps.CSR.from_host(items, dev), chunk_size=8192)
    qq = sps.prepare_queries(sps.CSR.from_host(q, dev), it)
    out = torch.empty(q.n_rows, 8192, dtype=torch.float32, device=dev)
    sums = torch.empty(it.num_chunks, q.n_rows, dtype=torch.float64, device=dev)
    sps.cosine_stream(qq, it, 0, it.num_chunks, out, sums)
    last = it.chunk_len(it.num_chunks - 1)
    b = (it.num_chunks - 1) * 8192
    assert float(np.abs(out[:, :last].cpu().numpy() - ref[:, b:]).max()) <= TOL
    s = sums.cpu().numpy()
    for c in range(it.num_chunks):
        n = it.chunk_len(c)
        assert np.abs(s[c] - ref[:, c * 8192:c * 8192 + n].sum(1)).max() <= 1e-4


def test_validate_and_bad_input(env):
    """sps_validate_csr names each fault; a structurally bad CSR is scored as
    empty by the prepare calls (no access outside the buffers)."""
    import pins
    from synth import HostCSR
    torch, sps, dev = env
    ok = pins.csr_from_rows([[(1, 1.0), (5, 2.0)], [], [(0, 3.0), (7, 1.0)]], 8)
    assert sps.validate_csr(sps.CSR.from_host(ok, dev)) == (True, -1, 0)
    cases = [
        (HostCSR(ok.indptr, np.array([5, 1, 0, 7], np.int32), ok.values, 3, 8), 0, 2),
        (HostCSR(ok.indptr, np.array([1, 5, 0, 9], np.int32), ok.values, 3, 8), 2, 3),
        (HostCSR(ok.indptr, ok.indices, np.array([1, 2, np.inf, 1], np.float32), 3, 8), 2, 4),
        (HostCSR(np.array([0, 3, 2, 4], np.int32), np.array([0, 1, 5, 7], np.int32),
                 ok.values, 3, 8), 1, 1),
    ]
    for m, row, why in cases:
        assert sps.validate_csr(sps.CSR.from_host(m, dev)) == (False, row, why)
    # an index outside [0, n_cols) in the items: prepared as empty, scored 0
    bad_items = HostCSR(ok.indptr, np.array([1, 5, 0, 99], np.int32), ok.values, 3, 8)
    it = sps.prepare(sps.CSR.from_host(bad_items, dev), chunk_size=2)
    qq = sps.prepare_queries(sps.CSR.from_host(ok, dev), it)
    out = torch.full((3, 2), float("nan"), device=dev)
    for c in range(it.num_chunks):
        sps.cosine_chunk(qq, it, c, out)
        assert torch.all(out[:, :it.chunk_len(c)] == 0).item()
    # and in the queries
    it = sps.prepare(sps.CSR.from_host(ok, dev), chunk_size=2)
    qq = sps.prepare_queries(sps.CSR.from_host(bad_items, dev), it)
    for c in range(it.num_chunks):
        out.fill_(float("nan"))
        sps.cosine_chunk(qq, it, c, out)
        assert torch.all(out[:, :it.chunk_len(c)] == 0).item()


def test_argument_errors(env):
    torch, sps, dev = env
    q, items, _ = synth.make_workload("tiny", n_item=100, n_query=4)
    it = sps.prepare(sps.CSR.from_host(items, dev), chunk_size=64)
    qq = sps.prepare_queries(sps.CSR.from_host(q, dev), it)
    out = torch.empty(4, 64, device=dev)
    with pytest.raises(sps.SpsError) as e:
        sps.cosine_chunk(qq, it, 2, out)
    assert e.value.status == -5
    other = synth.make_corpus(10, 999, 1, 0, nnz=("uniform", 1, 3), idx=("uniform",), val=0)
    with pytest.raises(sps.SpsError) as e:
        sps.prepare_queries(sps.CSR.from_host(other, dev), it)
    assert e.value.status == -3
    # a query batch is tied to the corpus it was prepared for
    it2 = sps.prepare(sps.CSR.from_host(items, dev), chunk_size=64)
    with pytest.raises(sps.SpsError) as e:
        sps.cosine_chunk(qq, it2, 0, out)
    assert e.value.status == -1
    # an output narrower than the chunk is refused (by the binding, then the library)
    with pytest.raises(AssertionError):
        sps.cosine_chunk(qq, it, 0, torch.empty(4, 63, device=dev))
    assert sps._lib.sps_cosine_chunk(qq._h, it._h, 0, out.data_ptr(), 63, None, None) == -1
