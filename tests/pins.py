"""Pins of the float64 oracle against facts that do not come from the oracle.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
on disagreement. They run against the real oracle (tests/test_oracle_pins.py)
and against deliberately broken builds of it (tests/test_oracle_mutants.py),
where at least one pin must fail for every planted mistake.

What each pin compares with:
* worked examples -- hand-derived closed forms of the cosine definition
  (tests/golden/worked_examples.json);
* brute force     -- densified float64 rows and numpy dot products (tiny dims);
* library routine -- scipy's sparse product of row-normalised matrices;
* invariants      -- self-similarity 1, symmetry, |S| <= 1, zero-norm rows 0,
  scale and sign, permutation of dims, duplicated rows;
* transpose       -- scipy's canonical CSR->CSC conversion;
* checksums       -- row and column sums of merged scores.
"""
from __future__ import annotations

import json
import os

import numpy as np

import synth
from synth import HostCSR

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "worked_examples.json")


def csr_from_rows(rows, n_cols) -> HostCSR:
    """rows: list of [(dim, value), ...] in any order -> canonical CSR."""
    indptr = [0]
    idx, val = [], []
    for r in rows:
        r = sorted(r, key=lambda t: t[0])
        idx += [int(t[0]) for t in r]
        val += [float(t[1]) for t in r]
        indptr.append(len(idx))
    return HostCSR(np.array(indptr, np.int32), np.array(idx, np.int32),
                   np.array(val, np.float32), len(rows), n_cols)


def random_csr(rng, n_rows, n_cols, lo, hi, *, signed=False, empty_frac=0.0,
               explicit_zero_frac=0.0) -> HostCSR:
    rows = []
    for _ in range(n_rows):
        k = int(rng.integers(lo, hi + 1))
        if rng.random() < empty_frac:
            k = 0
        d = rng.choice(n_cols, size=min(k, n_cols), replace=False)
        v = rng.standard_normal(len(d)) if signed else rng.lognormal(0, 1, len(d))
        if explicit_zero_frac:
            v[rng.random(len(d)) < explicit_zero_frac] = 0.0
        rows.append(list(zip(d.tolist(), v.astype(np.float32).tolist())))
    return csr_from_rows(rows, n_cols)


def dense64(m: HostCSR) -> np.ndarray:
    a = np.zeros((m.n_rows, m.n_cols), dtype=np.float64)
    for r in range(m.n_rows):
        d, v = m.row(r)
        a[r, d] = v.astype(np.float64)
    return a


def dense_cosine(q: HostCSR, i: HostCSR) -> np.ndarray:
    A, B = dense64(q), dense64(i)
    na = np.sqrt((A * A).sum(1))
    nb = np.sqrt((B * B).sum(1))
    dots = A @ B.T
    out = np.zeros_like(dots)
    ok = (na[:, None] > 0) & (nb[None, :] > 0)
    den = na[:, None] * nb[None, :]
    out[ok] = dots[ok] / den[ok]
    return out


# ---------------------------------------------------------------------------

def pin_worked_examples(orc):
    g = json.load(open(GOLDEN))
    for c in g["cases"]:
        q = csr_from_rows([c["u"]], 1200000)
        i = csr_from_rows([c["v"]], 1200000)
        s = orc.scores(q, i)[0, 0]
        assert abs(s - c["expected"]) <= 1e-15, (c["name"], s, c["expected"])
    for c in g["norms"]["cases"]:
        m = csr_from_rows([[(k, v) for k, v in enumerate(c["values"])]], 16)
        n64, inv = orc.row_norms(m)
        assert n64[0] == c["expected"], (c, n64[0])
        exp_inv = np.float32(1.0 / c["expected"]) if c["expected"] > 0 else np.float32(0)
        assert inv[0] == exp_inv, (c, inv[0])


def pin_bruteforce(orc, seed=11):
    rng = np.random.default_rng(seed)
    for n_cols, lo, hi, signed in [(64, 0, 12, False), (512, 1, 40, True), (4096, 0, 64, True)]:
        q = random_csr(rng, 23, n_cols, lo, hi, signed=signed, empty_frac=0.1,
                       explicit_zero_frac=0.05)
        i = random_csr(rng, 37, n_cols, lo, hi, signed=signed, empty_frac=0.1,
                       explicit_zero_frac=0.05)
        got = orc.scores(q, i)
        ref = dense_cosine(q, i)
        err = np.abs(got - ref).max()
        assert err <= 1e-13, ("bruteforce", n_cols, err)
        n64, _ = orc.row_norms(i)
        assert np.allclose(n64, np.sqrt((dense64(i) ** 2).sum(1)), rtol=1e-15, atol=0)


def pin_scipy(orc):
    from sklearn.preprocessing import normalize  # scipy-backed row normalisation
    q, i, _ = synth.make_workload("tiny")
    got = orc.scores(q, i)
    Q = q.to_scipy().astype(np.float64)
    I = i.to_scipy().astype(np.float64)
    ref = (normalize(Q) @ normalize(I).T).toarray()
    err = np.abs(got - ref).max()
    assert err <= 1e-12, ("scipy", err)
    # a signed, heavy-overlap sample too
    rng = np.random.default_rng(5)
    q = random_csr(rng, 40, 300, 1, 80, signed=True, empty_frac=0.05)
    i = random_csr(rng, 70, 300, 1, 80, signed=True, empty_frac=0.05)
    got = orc.scores(q, i)
    ref = (normalize(q.to_scipy().astype(np.float64)) @
           normalize(i.to_scipy().astype(np.float64)).T).toarray()
    assert np.abs(got - ref).max() <= 1e-12


def pin_invariants(orc, seed=3):
    rng = np.random.default_rng(seed)
    m = random_csr(rng, 60, 2000, 0, 50, signed=True, empty_frac=0.1)
    S = orc.scores(m, m)
    n64, _ = orc.row_norms(m)
    nz = n64 > 0
    # self-similarity is 1 for non-zero rows, exactly 0 for zero-norm rows
    d = np.diag(S)
    assert np.all(np.abs(d[nz] - 1.0) <= 1e-14), d[nz]
    assert np.all(S[~nz, :] == 0.0) and np.all(S[:, ~nz] == 0.0)
    # symmetry when queries equal items
    assert np.abs(S - S.T).max() <= 1e-15
    # range
    assert np.abs(S).max() <= 1.0 + 1e-12
    # disjoint supports give exactly 0
    a = csr_from_rows([[(2 * k, 1.5) for k in range(30)]], 100)
    b = csr_from_rows([[(2 * k + 1, -0.5) for k in range(30)]], 100)
    assert orc.scores(a, b)[0, 0] == 0.0
    # scale and sign: S(alpha u, beta v) = sign(alpha beta) S(u, v)
    q = random_csr(rng, 9, 500, 1, 40, signed=True)
    i = random_csr(rng, 13, 500, 1, 40, signed=True)
    base = orc.scores(q, i)
    for alpha, beta in [(4.0, 0.25), (-2.0, 8.0), (-0.5, -16.0)]:  # powers of two scale exactly
        q2 = HostCSR(q.indptr, q.indices, (q.values * np.float32(alpha)).astype(np.float32),
                     q.n_rows, q.n_cols)
        i2 = HostCSR(i.indptr, i.indices, (i.values * np.float32(beta)).astype(np.float32),
                     i.n_rows, i.n_cols)
        s2 = orc.scores(q2, i2)
        assert np.abs(s2 - np.sign(alpha * beta) * base).max() <= 1e-14
    # a consistent permutation of dims leaves S unchanged
    perm = rng.permutation(500)

    def permute(m):
        rows = []
        for r in range(m.n_rows):
            d, v = m.row(r)
            rows.append(list(zip(perm[d].tolist(), v.tolist())))
        return csr_from_rows(rows, m.n_cols)
    assert np.abs(orc.scores(permute(q), permute(i)) - base).max() <= 1e-15
    # duplicated item rows give identical columns
    dup = i.take_rows([0, 1, 0, 2, 1])
    sd = orc.scores(q, dup)
    assert np.array_equal(sd[:, 0], sd[:, 2]) and np.array_equal(sd[:, 1], sd[:, 4])


def pin_csc(orc):
    import scipy.sparse as sp
    q, items, _ = synth.make_workload("mid", n_item=20000, n_query=8)
    n64, _ = orc.row_norms(items)
    C = 8192
    for c, (b, e) in enumerate([(0, C), (C, 2 * C), (2 * C, items.n_rows)]):
        col_ptr, row, val = orc.chunk_csc(items, n64, b, e)
        p0, p1 = int(items.indptr[b]), int(items.indptr[e])
        sub = sp.csr_matrix((items.values[p0:p1].astype(np.float64), items.indices[p0:p1],
                             (items.indptr[b:e + 1] - items.indptr[b])),
                            shape=(e - b, items.n_cols))
        T = sub.tocsc()
        T.sort_indices()
        assert np.array_equal(col_ptr, T.indptr.astype(np.int32)), c
        assert np.array_equal(row, T.indices.astype(np.int32)), c
        exp = (T.data / n64[b + T.indices]).astype(np.float32)
        assert np.array_equal(val, exp), c
        # invariants: monotone, total, back-transpose reproduces the chunk
        assert col_ptr[0] == 0 and col_ptr[-1] == p1 - p0 and np.all(np.diff(col_ptr) >= 0)
        back = sp.csc_matrix((np.ones_like(val), row, col_ptr),
                             shape=(e - b, items.n_cols)).tocsr()
        back.sort_indices()
        assert np.array_equal(back.indices, items.indices[p0:p1])
        assert np.array_equal(back.indptr, items.indptr[b:e + 1] - items.indptr[b])


def pin_checksums(orc):
    rng = np.random.default_rng(21)
    q = random_csr(rng, 31, 700, 0, 60, signed=True, empty_frac=0.1)
    items = random_csr(rng, 1000, 700, 0, 60, signed=True, empty_frac=0.1)
    S = orc.scores(q, items)
    C = 384
    rs = orc.chunk_row_sums(q, items, C)
    assert rs.shape == (3, q.n_rows)
    for c in range(3):
        b, e = c * C, min((c + 1) * C, items.n_rows)
        assert np.abs(rs[c] - S[:, b:e].sum(1)).max() <= 1e-9
    cs = orc.col_sums(q, items, 100, 900)
    assert np.abs(cs - S[:, 100:900].sum(0)).max() <= 1e-9
    # the same closed forms over |q^_d i^_d| and over shared-dim counts, against
    # brute-force densified rows: |Q^| |I^|^T and the product of the stored-entry masks
    qn, _ = orc.row_norms(q)
    inn, _ = orc.row_norms(items)
    dq, di = dense64(q), dense64(items)
    qh = np.where(qn[:, None] > 0, dq / np.where(qn > 0, qn, 1.0)[:, None], 0.0)
    ih = np.where(inn[:, None] > 0, di / np.where(inn > 0, inn, 1.0)[:, None], 0.0)

    def mask(m, nrm):
        z = np.zeros((m.n_rows, m.n_cols))
        for r in range(m.n_rows):
            if nrm[r] > 0:
                z[r, m.indices[m.indptr[r]:m.indptr[r + 1]]] = 1.0
        return z
    A = np.abs(qh) @ np.abs(ih).T
    M = mask(q, qn) @ mask(items, inn).T
    rs1 = orc.chunk_row_sums(q, items, C, kind=1)
    rs2 = orc.chunk_row_sums(q, items, C, kind=2)
    for c in range(3):
        b, e = c * C, min((c + 1) * C, items.n_rows)
        assert np.abs(rs1[c] - A[:, b:e].sum(1)).max() <= 1e-9
        assert np.array_equal(rs2[c], M[:, b:e].sum(1))
    assert np.abs(orc.col_sums(q, items, 100, 900, kind=1) - A[:, 100:900].sum(0)).max() <= 1e-9
    assert np.array_equal(orc.col_sums(q, items, 100, 900, kind=2), M[:, 100:900].sum(0))
    # |S| <= the absolute sum (termwise), with equality for the non-negative pairs
    assert np.all(np.abs(S) <= A + 1e-12)


ALL_PINS = [pin_worked_examples, pin_bruteforce, pin_scipy, pin_invariants, pin_csc,
            pin_checksums]
