"""The streaming loop with the output on the host: each chunk's scores go into
a host output matrix (§2.2 and §4.4 of "稀疏嵌入批量相似度计算的工程化实践"),
here through two alternating device buffers and the copy engine, through the
C ABI.

The host matrix must equal the device chunk outputs bit for bit (those are
within 1e-5 of the float64 oracle, as test_gpu_parity.py shows); sampled rows
are also compared with the oracle directly.
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


def _device_chunks(env, it, qq, n_q, chunks):
    """{chunk: (fp32 scores [n_q, chunk_len] on the host, row sums)} by sps_cosine_chunk."""
    torch, sps, dev = env
    out = torch.empty(n_q, max(min(it.chunk_size, it.n_items), 1), dtype=torch.float32,
                      device=dev)
    rs = torch.empty(n_q, dtype=torch.float64, device=dev)
    res = {}
    for c in chunks:
        sps.cosine_chunk(qq, it, c, out, rs)
        res[c] = (out[:, :it.chunk_len(c)].cpu().numpy().copy(), rs.cpu().numpy().copy())
    return res


def test_host_stream_mid_all_chunks(env, orc):
    torch, sps, dev = env
    q, items, _ = synth.make_workload("mid")
    it, qq = _prepared(env, q, items, 8192)
    host = torch.empty(q.n_rows, items.n_rows, dtype=torch.float32, pin_memory=True)
    sums = torch.empty(it.num_chunks, q.n_rows, dtype=torch.float64, device=dev)
    sps.cosine_stream_host(qq, it, 0, it.num_chunks, host, row_sums=sums)
    torch.cuda.synchronize()
    h = host.numpy()
    ref = _device_chunks(env, it, qq, q.n_rows, range(it.num_chunks))
    for c, (d, rs) in ref.items():
        b = c * 8192
        assert np.array_equal(h[:, b:b + d.shape[1]].view(np.uint32), d.view(np.uint32)), c
        assert np.array_equal(sums[c].cpu().numpy(), rs)
    rows = np.sort(np.random.default_rng(5).choice(q.n_rows, 16, replace=False))
    err = float(np.abs(h[rows] - orc.scores(q, items, q_rows=rows)).max())
    assert err < TOL
    report("host stream mid 2000x100000, 13 chunks: bit-equal to the device chunks; "
           "16 rows vs oracle max|err|=%.3g" % err)


def test_host_stream_ragged_range_and_pitches(env, orc):
    """A chunk range not starting at 0 that ends with the partial last chunk, a host
    pitch wider than the range (the extra columns untouched), a device pitch wider
    than the chunk, a one-chunk range, and an empty one."""
    torch, sps, dev = env
    q, items, _ = synth.make_workload("edge", n_item=30000, n_query=300)
    C = 4097
    it, qq = _prepared(env, q, items, C)
    assert it.num_chunks == 8 and it.chunk_len(7) == 30000 - 7 * C
    cb, ce = 3, 8
    span = items.n_rows - cb * C
    host = torch.full((q.n_rows, span + 37), float("nan"), dtype=torch.float32,
                      pin_memory=True)
    bufs = tuple(torch.empty(q.n_rows, C + 11, dtype=torch.float32, device=dev)
                 for _ in range(2))
    sums = torch.empty(ce - cb, q.n_rows, dtype=torch.float64, device=dev)
    sps.cosine_stream_host(qq, it, cb, ce, host, bufs=bufs, row_sums=sums)
    torch.cuda.synchronize()
    h = host.numpy()
    ref = _device_chunks(env, it, qq, q.n_rows, range(cb, ce))
    for c, (d, rs) in ref.items():
        b = (c - cb) * C
        assert np.array_equal(h[:, b:b + d.shape[1]].view(np.uint32), d.view(np.uint32)), c
        assert np.array_equal(sums[c - cb].cpu().numpy(), rs)
    assert np.all(np.isnan(h[:, span:]))
    ref_o = orc.scores(q, items, item_begin=cb * C, item_end=items.n_rows)
    err = float(np.abs(h[:, :span] - ref_o).max())
    assert err < TOL
    # one chunk; an empty range leaves everything untouched
    one = torch.full((q.n_rows, C), float("nan"), dtype=torch.float32, pin_memory=True)
    sps.cosine_stream_host(qq, it, 5, 6, one, bufs=bufs)
    sps.cosine_stream_host(qq, it, 6, 6, one, bufs=bufs)
    torch.cuda.synchronize()
    assert np.array_equal(one.numpy().view(np.uint32), ref[5][0].view(np.uint32))
    report("host stream edge 300x30000, chunks [3, 8) of 4097 (partial last), "
           "ld_host + 37, ld_dev + 11: bit-equal; vs oracle max|err|=%.3g" % err)


def test_host_stream_pages_full_size(env):
    """Full pages shape in the benchmark's chunking: the last two chunks (one full,
    one partial) into pinned host memory, bit-equal to the device chunks."""
    torch, sps, dev = env
    q, items, _ = synth.make_workload("pages")
    it, qq = _prepared(env, q, items, 8192)
    cb, ce = it.num_chunks - 2, it.num_chunks
    span = items.n_rows - cb * 8192
    host = torch.empty(q.n_rows, span, dtype=torch.float32, pin_memory=True)
    sps.cosine_stream_host(qq, it, cb, ce, host)
    torch.cuda.synchronize()
    h = host.numpy()
    ref = _device_chunks(env, it, qq, q.n_rows, range(cb, ce))
    for c, (d, _) in ref.items():
        b = (c - cb) * 8192
        assert np.array_equal(h[:, b:b + d.shape[1]].view(np.uint32), d.view(np.uint32)), c
    report("host stream pages chunks [%d, %d): %d x %d bit-equal to the device chunks"
           % (cb, ce, q.n_rows, span))


def test_bulk_similarity_pinned_host(env):
    torch, sps, dev = env
    q, items, _ = synth.make_workload("tiny")
    dq, di = sps.CSR.from_host(q, dev), sps.CSR.from_host(items, dev)
    on_dev = sps.bulk_similarity(dq, di, chunk_size=1000)
    host = torch.empty(q.n_rows, items.n_rows, dtype=torch.float32, pin_memory=True)
    sps.bulk_similarity(dq, di, chunk_size=1000, out=host)
    assert torch.equal(on_dev.cpu(), host)


def test_host_stream_arguments(env):
    torch, sps, dev = env
    q, items, _ = synth.make_workload("tiny", n_item=3000, n_query=7)
    it, qq = _prepared(env, q, items, 1024)
    bufs = tuple(torch.empty(7, 1024, dtype=torch.float32, device=dev) for _ in range(2))
    pinned = torch.empty(7, 3000, dtype=torch.float32, pin_memory=True)
    lib = sps._lib
    s = torch.cuda.current_stream().cuda_stream
    cs = sps._copy_stream(dev).cuda_stream

    def call(host_ptr, ld_host, b0, b1, ld_dev=1024, cb=0, ce=3):
        return lib.sps_cosine_stream_host(qq._h, it._h, cb, ce, host_ptr, ld_host, b0, b1,
                                          ld_dev, None, s, cs)
    p0, p1 = bufs[0].data_ptr(), bufs[1].data_ptr()
    # pageable host memory is refused (the copy engine would not overlap)
    pageable = np.empty((7, 3000), dtype=np.float32)
    assert call(pageable.ctypes.data, 3000, p0, p1) == -1
    assert call(pinned.data_ptr(), 3000, p0, p0) == -1       # the same buffer twice
    assert call(pinned.data_ptr(), 3000, p0, None) == -1     # one buffer
    assert call(pinned.data_ptr(), 2999, p0, p1) == -1       # host pitch below the range
    assert call(pinned.data_ptr(), 3000, p0, p1, ld_dev=1023) == -1
    assert call(None, 3000, p0, p1) == -1
    assert call(pinned.data_ptr(), 3000, p0, p1, cb=2, ce=4) == -5
    assert call(pinned.data_ptr(), 3000, p0, p1, cb=2, ce=1) == -5
    # nothing was enqueued by the refused calls; a good call still works
    assert call(pinned.data_ptr(), 3000, p0, p1) == 0
    torch.cuda.synchronize()
    assert torch.isfinite(pinned).all()
