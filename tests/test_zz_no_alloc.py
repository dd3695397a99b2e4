"""sps_cosine_chunk_static (partial row sums in the library's static device
scratch, no allocation) against sps_cosine_chunk, through the C ABI.

Two workloads in a row, the second smaller, so the second call runs on a
scratch that still holds the first call's partial sums; scores and row sums
must be bitwise equal to the existing entry point's, which the parity tests
hold to the float64 oracle."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_embedding_exact_amd as sps
    sps.load_library()
    return torch, sps, torch.device("cuda:0")


def _compare(env, q, items, chunk_size):
    torch, sps, dev = env
    it = sps.prepare(sps.CSR.from_host(items, dev), chunk_size=chunk_size)
    qq = sps.prepare_queries(sps.CSR.from_host(q, dev), it)
    width = min(chunk_size, items.n_rows)
    a = torch.empty(q.n_rows, width, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    ra = torch.empty(q.n_rows, dtype=torch.float64, device=dev)
    rb = torch.empty_like(ra)
    for c in range(it.num_chunks):
        n = it.chunk_len(c)
        a.fill_(float("nan"))
        b.fill_(float("nan"))
        sps.cosine_chunk(qq, it, c, a, ra)
        sps.cosine_chunk_static(qq, it, c, b, rb)
        torch.cuda.synchronize()
        assert torch.equal(a[:, :n].view(torch.int32), b[:, :n].view(torch.int32)), c
        assert torch.equal(ra.view(torch.int64), rb.view(torch.int64)), c
        # without row sums too
        b.fill_(float("nan"))
        sps.cosine_chunk_static(qq, it, c, b)
        torch.cuda.synchronize()
        assert torch.equal(a[:, :n].view(torch.int32), b[:, :n].view(torch.int32)), c
    return it.num_chunks


def test_static_scratch_matches_two_calls(env):
    q, items, _ = synth.make_workload("mid", n_item=30000, n_query=2000)
    assert _compare(env, q, items, 8192) == 4  # 8 slices per chunk: partial sums in scratch
    q, items, _ = synth.make_workload("edge", n_item=9001, n_query=300)
    assert _compare(env, q, items, 4096) == 3  # smaller: 4 slices, 300 rows


def test_static_scratch_limit(env):
    torch, sps, dev = env
    q, items, _ = synth.make_workload("tiny", n_item=8192, n_query=65537)
    rs = torch.empty(q.n_rows, dtype=torch.float64, device=dev)
    ref = torch.empty_like(rs)
    # 2 slices per chunk: 131074 doubles of scratch, within the 524288 limit
    it = sps.prepare(sps.CSR.from_host(items, dev), chunk_size=2048)
    qq = sps.prepare_queries(sps.CSR.from_host(q, dev), it)
    out = torch.empty(q.n_rows, 2048, dtype=torch.float32, device=dev)
    sps.cosine_chunk_static(qq, it, 1, out, rs)
    sps.cosine_chunk(qq, it, 1, out, ref)
    torch.cuda.synchronize()
    assert torch.equal(rs.view(torch.int64), ref.view(torch.int64))
    # 8 slices per chunk: 65537 x 8 = 524296 doubles, beyond the limit
    it8 = sps.prepare(sps.CSR.from_host(items, dev), chunk_size=8192)
    qq8 = sps.prepare_queries(sps.CSR.from_host(q, dev), it8)
    out8 = torch.empty(q.n_rows, 8192, dtype=torch.float32, device=dev)
    with pytest.raises(sps.SpsError) as e:
        sps.cosine_chunk_static(qq8, it8, 0, out8, rs)
    assert e.value.status == -8 and "static scratch" in str(e.value)
    sps.cosine_chunk_static(qq8, it8, 0, out8)  # no row sums: no scratch needed
    torch.cuda.synchronize()
