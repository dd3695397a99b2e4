#!/usr/bin/env python3
"""Throughput of the exact sparse-cosine path on one MI355X.

One step = the whole path over the workload: item norms + per-chunk
inverted lists (sps_prepare), query norms + row groups
(sps_prepare_queries), then every item chunk scored into one rotating
(n_query x 8192) float32 device buffer with a float64 row-sum checksum per
chunk (the streaming loop of §2.2 / §4.4 of "稀疏嵌入批量相似度计算的工程化实践").
Inputs are seeded synthetic CSR already resident in HBM when timing starts.

Prints one JSON line: scores/s over the timed steps, the score kernel's
achieved algorithmic HBM bandwidth against the 8 TB/s peak (HIP events
around every score launch, on the stream the kernels run on), and the
float64 CPU oracle timed on a bounded sample of the same workload. The
reduced-precision variant (fp16 item values and scores, |error| < 1e-3, as
§5.3 of the page allows) is timed the same way and reported under
"variants", and so is the threshold-filtered output (the exact scores >= t,
t = 0.5 unless --threshold says otherwise, appended as (row, item, score)
hits), and so is the output streamed into pinned host memory (the first
--host-chunks chunks, against a plain device-to-host copy's rate) and the
Block-Sparse CSR form of the item corpus (index bytes, encode and decode
times); none of them ever stands in for the exact path's value.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="pages", help="tiny|mid|pages|dense|edge")
    ap.add_argument("--cpu-rows", type=int, default=384,
                    help="query rows of the oracle sample (x all items)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-half", action="store_true",
                    help="skip the fp16 reduced-precision variant's timing")
    ap.add_argument("--threshold", type=float, default=0.5,
                    help="score threshold of the threshold-filtered variant's timing")
    ap.add_argument("--no-threshold", dest="threshold", action="store_const", const=None,
                    help="skip the threshold-filtered variant's timing")
    ap.add_argument("--host-chunks", type=int, default=4,
                    help="chunks streamed into pinned host memory for the host-output "
                         "variant's timing (0 skips it)")
    ap.add_argument("--no-bsc", action="store_true",
                    help="skip the Block-Sparse CSR codec's timing")
    ap.add_argument("--configs", default="tiny,mid,dense,edge",
                    help="other workloads whose score launches are timed and reported under "
                         "variants.configs (comma list; '' skips)")
    ap.add_argument("--no-dense-ab", action="store_true",
                    help="skip the timing of the path with the heavy-dim matrix-core part off "
                         "(SPS_DENSE=0) on pages and dense")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles",
                                                      "score_kernel_pages_traffic.txt"),
                    help="measured HBM bytes per score launch (rocprofv3 FETCH_SIZE / "
                         "WRITE_SIZE summary); used only while the score kernel's sources "
                         "still hash to the value recorded there")
    ap.add_argument("--event-every", type=int, default=16, metavar="E",
                    help="timed steps bracket every E-th score launch with events (step k "
                         "the chunks c = k mod E), for the average launch duration; a "
                         "per-launch event pair costs about 6 us of a step, so 1 (every "
                         "launch) adds about 1.5 ms to the pages step")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (5 times) and "
                         "exit: the reference for scaling FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


SCORE_SOURCES = ("sps_score.hip", "sps_internal.h", "sps_device.h")


def score_source_hash():
    """SHA-256 over the score kernel's sources (the counters describe that code only)."""
    import hashlib
    h = hashlib.sha256()
    for name in SCORE_SOURCES:
        with open(os.path.join(ROOT, "sparse_embedding_exact_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(path, workload):
    """HBM bytes per score launch from a committed counter summary ("key: value" lines), or
    None when there is none for this workload or the kernel changed since it was taken."""
    if not path or not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.lstrip().startswith(("#", "|", "`")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("workload") != workload or kv.get("source_sha256") != score_source_hash():
        return None
    try:
        return float(kv["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def host_cpus():
    """CPU model, the affinity mask, this process's CPU share (cgroup quota, and
    OMP_NUM_THREADS where the job sets it), and the cores one pinned thread each
    should use: the first `share` cores of the mask."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    mask = sorted(os.sched_getaffinity(0))
    quota = None
    for path, parse_q in (("/sys/fs/cgroup/cpu.max", lambda t: t.split()),
                          ("/sys/fs/cgroup/cpu/cpu.cfs_quota_us", None)):
        try:
            with open(path) as f:
                txt = f.read().strip()
        except OSError:
            continue
        if parse_q is not None:
            q, per = parse_q(txt)
            if q != "max":
                quota = max(1, int(int(q) // int(per)))
        else:
            try:
                with open("/sys/fs/cgroup/cpu/cpu.cfs_period_us") as f:
                    per = int(f.read())
                if int(txt) > 0:
                    quota = max(1, int(txt) // per)
            except (OSError, ValueError):
                pass
        break
    omp = os.environ.get("OMP_NUM_THREADS")
    share = len(mask)
    if quota:
        share = min(share, quota)
    if omp and omp.isdigit() and int(omp) > 0:
        share = min(share, int(omp))
    return {"cpu_model": model, "affinity_cores": len(mask), "cgroup_cpu_quota": quota,
            "omp_num_threads": omp, "cores_used": mask[:share]}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (item chunks "
              "would be sharded across GPUs, each scoring its own chunks with no collective "
              "in the hot loop). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_probe:
        n = args.copy_probe * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": 4 * n, "launches": 5}))
        return

    import sparse_embedding_exact_amd as sps
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sps.load_library()
    w = synth.WORKLOADS[args.workload]

    t0 = time.time()
    q_host, i_host, _ = synth.make_workload(w)
    log("generated %s in %.1fs: items nnz %d, queries nnz %d" %
        (w.name, time.time() - t0, i_host.nnz, q_host.nnz))
    items = sps.CSR.from_host(i_host, dev)
    queries = sps.CSR.from_host(q_host, dev)
    C = w.chunk_size
    n_q, n_i = q_host.n_rows, i_host.n_rows
    out = torch.empty(n_q, min(C, n_i), dtype=torch.float32, device=dev)
    n_chunks = (n_i + C - 1) // C
    sums = torch.empty(n_chunks, n_q, dtype=torch.float64, device=dev)
    chunk_nnz = np.diff(i_host.indptr[np.minimum(np.arange(n_chunks + 1) * C, n_i)])
    chunk_len = np.minimum(C, n_i - np.arange(n_chunks) * C)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def pair():
        return (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))

    def make_step(score_chunk, half=False, before=None):
        """One pass of the path: prepare items and queries, then score every chunk.
        `evs` (timed steps only) holds the step's own events: (step, prepare, score
        loop, {chunk: pair} for the sampled chunks)."""
        def step(evs=None):
            if evs is not None:
                evs[0][0].record(stream)
            if before is not None:
                before()
            if evs is not None:
                evs[1][0].record(stream)
            it = sps.prepare(items, chunk_size=C)
            if half:
                it.enable_half()
            qq = sps.prepare_queries(queries, it)
            if evs is not None:
                evs[1][1].record(stream)
                evs[2][0].record(stream)
            for c in range(n_chunks):
                e = evs[3].get(c) if evs is not None else None
                if e is not None:
                    e[0].record(stream)
                score_chunk(qq, it, c)
                if e is not None:
                    e[1].record(stream)
            if evs is not None:
                evs[2][1].record(stream)
                evs[0][1].record(stream)
            return it, qq
        return step

    def sampled_chunks(k):
        """The chunks whose launches timed step k brackets with events."""
        e = max(1, args.event_every)
        r = (k % e) % n_chunks
        return [c for c in range(n_chunks) if c % e == r]

    class Timed:
        """A timed run: wall seconds over the steps, the sampled launches' (chunk,
        ms) pairs, the mean prepare and score-loop ms per step, the median step ms."""
        def __init__(self, total, samples, prep, loop, median):
            self.total, self.samples, self.prep, self.loop, self.median = (
                total, samples, prep, loop, median)

        def launch_ms(self):
            return np.array([ms for _, ms in self.samples])

        def avg_launch_ms(self):
            return float(self.launch_ms().mean())

        def achieved_gbps(self, nbytes):
            """Algorithmic bytes of the sampled launches over their summed time."""
            b = float(sum(nbytes[c] for c, _ in self.samples))
            return b / (float(self.launch_ms().sum()) * 1e-3) / 1e9

    def run_timed(step):
        """Warmup, then exactly args.steps timed steps, bracketed by a synchronize on
        both sides and nothing else between them. Every timed step records events
        of its own (the step, the prepare, the score loop, and the sampled chunks'
        launches), read only after the timed region, so that reading them is not
        timed; the median step is taken from the steps' own events."""
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        evs = [(pair(), pair(), pair(), {c: pair() for c in sampled_chunks(k)})
               for k in range(args.steps)]
        t0 = time.perf_counter()
        for k in range(args.steps):
            # (a step's prepared structures are released as soon as its work is
            # queued: their workspaces are stream-ordered torch memory, reused by
            # the next step without new device allocations)
            step(evs[k])
        torch.cuda.synchronize()
        t_total = time.perf_counter() - t0
        samples, prep, loop, per_step = [], 0.0, 0.0, []
        for e_step, e_prep, e_loop, e_chunks in evs:
            samples += [(c, a.elapsed_time(b)) for c, (a, b) in sorted(e_chunks.items())]
            prep += e_prep[0].elapsed_time(e_prep[1])
            loop += e_loop[0].elapsed_time(e_loop[1])
            per_step.append(e_step[0].elapsed_time(e_step[1]))
        return Timed(t_total, samples, prep / args.steps, loop / args.steps,
                     float(np.median(per_step)))

    main = run_timed(make_step(lambda qq, it, c: sps.cosine_chunk(qq, it, c, out, sums[c])))
    t_total, prep_ms = main.total, main.prep
    ms_per_step = 1e3 * t_total / args.steps
    median_step_ms = main.median
    scores = float(n_q) * float(n_i)
    value = scores * args.steps / t_total

    # algorithmic bytes of one score launch: fp32 scores written, the chunk's
    # posting entries read once (8-byte (item id, value) records), fp64 row sums
    alg_bytes = 4.0 * n_q * chunk_len + 8.0 * chunk_nnz + 8.0 * n_q
    avg_launch_ms = main.avg_launch_ms()
    achieved = main.achieved_gbps(alg_bytes)
    loop_ms = main.loop
    traffic = measured_traffic(args.traffic, w.name)

    # checksum sanity on the last step: row sums finite
    assert torch.isfinite(sums).all().item()

    # a write-only ceiling for the same bytes: the output buffer zero-filled
    # (torch's fill kernel), timed with events on the same stream
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out.zero_()
    w0.record(stream)
    for _ in range(5):
        out.zero_()
    w1.record(stream)
    torch.cuda.synchronize()
    write_ceiling = 5 * 4.0 * out.numel() / (w0.elapsed_time(w1) * 1e-3) / 1e9
    log("step %.2f ms: prepare %.2f ms, %d score launches %.2f ms (avg %.3f ms)" %
        (ms_per_step, prep_ms, n_chunks, loop_ms, avg_launch_ms))

    def variant(tm, nbytes, **extra):
        avg = tm.avg_launch_ms()
        ach = tm.achieved_gbps(nbytes)
        d = {"value": scores * args.steps / tm.total, "unit": "scores/s",
             "ms_per_step": 1e3 * tm.total / args.steps}
        d.update(extra)
        d["breakdown_ms"] = {"prepare": tm.prep, "score_loop": tm.loop,
                             "score_launch_avg": avg}
        d["roofline"] = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": ach / HBM_PEAK_GBPS}
        return d

    # the reduced-precision variant (fp16 item values and scores, |error| < 1e-3),
    # timed the same way; reported beside the exact path, never as `value`
    half = None
    if not args.no_half:
        out16 = torch.empty(n_q, min(C, n_i), dtype=torch.float16, device=dev)
        h_tm = run_timed(make_step(
            lambda qq, it, c: sps.cosine_chunk_half(qq, it, c, out16, sums[c]), half=True))
        half = variant(h_tm, 2.0 * n_q * chunk_len + 4.0 * chunk_nnz + 8.0 * n_q,
                       dtype="f16", max_abs_error_bound=1e-3)
        log("fp16 variant: step %.2f ms, avg launch %.3f ms" %
            (half["ms_per_step"], half["breakdown_ms"]["score_launch_avg"]))

    # threshold-filtered output: the exact scores >= t appended as 12-byte hits;
    # an untimed counting pass (capacity 0) sizes the hit buffer, so no hit of a
    # timed step is dropped
    thr = None
    if args.threshold is not None:
        t_ = float(args.threshold)
        count = torch.zeros(1, dtype=torch.int64, device=dev)
        no_hits = torch.empty(0, 3, dtype=torch.int32, device=dev)
        count_step = make_step(
            lambda qq, it, c: sps.cosine_chunk_threshold(qq, it, c, t_, no_hits, count, sums[c]),
            before=count.zero_)
        count_step()
        torch.cuda.synchronize()
        n_hits = int(count.item())
        hits = torch.empty(n_hits, 3, dtype=torch.int32, device=dev)
        t_tm = run_timed(make_step(
            lambda qq, it, c: sps.cosine_chunk_threshold(qq, it, c, t_, hits, count, sums[c]),
            before=count.zero_))
        assert int(count.item()) == n_hits
        thr = variant(t_tm, 8.0 * chunk_nnz + 8.0 * n_q + 12.0 * n_hits / n_chunks,
                      dtype="f32", threshold=t_, hits=n_hits)
        log("threshold %.2f variant: %d hits, step %.2f ms, avg launch %.3f ms" %
            (t_, n_hits, thr["ms_per_step"], thr["breakdown_ms"]["score_launch_avg"]))

    # the output streamed to pinned host memory (double-buffered, the copy
    # engine on a side stream): `host_chunks` chunks after one prepare, against a
    # plain device-to-host copy of one chunk's bytes, the link's own rate
    host = None
    if args.host_chunks > 0:
        K = min(args.host_chunks, n_chunks)
        span = min(K * C, n_i)
        hout = torch.empty(n_q, span, dtype=torch.float32, pin_memory=True)
        it_h = sps.prepare(items, chunk_size=C)
        qq_h = sps.prepare_queries(queries, it_h)
        sps.cosine_stream_host(qq_h, it_h, 0, K, hout)  # warm-up
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            sps.cosine_stream_host(qq_h, it_h, 0, K, hout)
        torch.cuda.synchronize()
        hs = (time.perf_counter() - t0) / args.steps
        probe = torch.empty(n_q, min(C, n_i), dtype=torch.float32, device=dev)
        probe_h = torch.empty(n_q, min(C, n_i), dtype=torch.float32, pin_memory=True)
        probe_h.copy_(probe, non_blocking=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            probe_h.copy_(probe, non_blocking=True)
        torch.cuda.synchronize()
        cs = (time.perf_counter() - t0) / args.steps
        link = 4.0 * probe.numel() / cs / 1e9
        rate = 4.0 * n_q * span / hs / 1e9
        host = {"value": float(n_q) * span / hs, "unit": "scores/s", "dtype": "f32",
                "chunks": K, "ms_per_range": 1e3 * hs, "ms_per_chunk": 1e3 * hs / K,
                "d2h_gbps": rate, "plain_d2h_copy_gbps": link, "frac_of_plain_copy": rate / link,
                "note": "prepare excluded; the full %d-chunk matrix (%.0f GB) would take %.1f s "
                        "at this rate" % (n_chunks, 4.0 * n_q * n_i / 1e9, 4.0 * n_q * n_i / 1e9 / rate)}
        del hout, probe, probe_h, it_h, qq_h
        log("host stream: %d chunks in %.1f ms (%.1f GB/s; plain D2H copy %.1f GB/s)" %
            (K, 1e3 * hs, rate, link))

    # Block-Sparse CSR (compressed column indices) of the item corpus: index bytes
    # against CSR's, the encoder's time, and the device decode that precedes a prepare
    bscv = None
    if not args.no_bsc:
        t0 = time.perf_counter()
        bz = sps.bsc_encode(items)  # synchronises once to size the varint stream
        torch.cuda.synchronize()
        enc_ms = 1e3 * (time.perf_counter() - t0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        sps.bsc_decode(bz, check=True)  # warm-up, and a well-formed check
        reps = 10
        e0.record(stream)
        for _ in range(reps):
            sps.bsc_decode(bz, check=False)
        e1.record(stream)
        torch.cuda.synchronize()
        dec_ms = e0.elapsed_time(e1) / reps
        nnz_i = int(i_host.nnz)
        dec_bytes = 8.0 * (n_i + 1) + bz.blocks.numel() + (10 * nnz_i + 7) // 8 + 4.0 * nnz_i
        bscv = {"index_bytes_per_entry": bz.index_bytes() / nnz_i,
                "csr_index_bytes_per_entry": 4.0,
                "index_saving": 1.0 - bz.index_bytes() / (4.0 * nnz_i),
                "encode_ms": enc_ms, "decode_ms": dec_ms,
                "roofline": {"bound": "hbm", "achieved": dec_bytes / (dec_ms * 1e-3) / 1e9,
                             "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                             "frac": dec_bytes / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}}
        del bz
        log("bsc: %.3f index bytes per entry (CSR 4), encode %.1f ms, decode %.3f ms" %
            (bscv["index_bytes_per_entry"], enc_ms, dec_ms))

    # ---- other workloads: every chunk's score launch, events around each ----
    def time_chunks(qh, ih, C, reps=2, dense=None):
        """Prepare once (optionally with the heavy-dim part forced on or off), then time
        each chunk's score launch: per-launch ms (mean of `reps` passes after a warm-up
        pass), prepare ms, algorithmic bytes per launch."""
        old = os.environ.get("SPS_DENSE")
        if dense is not None:
            os.environ["SPS_DENSE"] = "1" if dense else "0"
        try:
            ci, cq = sps.CSR.from_host(ih, dev), sps.CSR.from_host(qh, dev)
            p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            p0.record(stream)
            it = sps.prepare(ci, chunk_size=C)
            qq = sps.prepare_queries(cq, it)
            p1.record(stream)
        finally:
            if old is None:
                os.environ.pop("SPS_DENSE", None)
            else:
                os.environ["SPS_DENSE"] = old
        nch = it.num_chunks
        o = torch.empty(qh.n_rows, min(C, ih.n_rows), dtype=torch.float32, device=dev)
        rs = torch.empty(qh.n_rows, dtype=torch.float64, device=dev)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(nch)]
        for c in range(nch):
            sps.cosine_chunk(qq, it, c, o, rs)
        torch.cuda.synchronize()
        prep = p0.elapsed_time(p1)
        kern = np.zeros(nch)
        for _ in range(reps):
            for c in range(nch):
                evs[c][0].record(stream)
                sps.cosine_chunk(qq, it, c, o, rs)
                evs[c][1].record(stream)
            torch.cuda.synchronize()
            kern += np.array([x.elapsed_time(y) for x, y in evs])
        clen = np.minimum(C, ih.n_rows - np.arange(nch) * C)
        cnnz = np.diff(ih.indptr[np.minimum(np.arange(nch + 1) * C, ih.n_rows)])
        alg = 4.0 * qh.n_rows * clen + 8.0 * cnnz + 8.0 * qh.n_rows
        del it, qq, ci, cq, o, rs
        return kern / reps, prep, alg

    def summary(kern, prep, alg, nq, ni):
        avg = float(kern.mean())
        ach = float(alg.mean()) / (avg * 1e-3) / 1e9
        return {"scores": float(nq) * ni, "chunks": int(len(kern)), "ms_per_launch": avg,
                "score_loop_ms": float(kern.sum()), "prepare_ms": prep,
                "scores_per_s": float(nq) * ni / (float(kern.sum()) * 1e-3),
                "alg_bytes_per_launch": float(alg.mean()),
                "floor_ms_per_launch": float(alg.mean()) / (HBM_PEAK_GBPS * 1e9) * 1e3,
                "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBPS,
                             "unit": "GB/s", "frac": ach / HBM_PEAK_GBPS}}

    configs = {}
    for name in [x for x in args.configs.split(",") if x and x != w.name]:
        wc = synth.WORKLOADS[name]
        qc, ic, _ = synth.make_workload(wc)
        k, pr, al = time_chunks(qc, ic, wc.chunk_size)
        configs[name] = summary(k, pr, al, qc.n_rows, ic.n_rows)
        configs[name]["workload"] = "%s: %s" % (wc.name, wc.description)
        log("config %s: %d launches, avg %.4f ms (%.1f%% of the HBM roofline), prepare %.2f ms"
            % (name, len(k), k.mean(), 100 * configs[name]["roofline"]["frac"], pr))
        if name == "dense" and not args.no_dense_ab:
            k0, pr0, al0 = time_chunks(qc, ic, wc.chunk_size, dense=False)
            configs[name]["heavy_dims_off"] = summary(k0, pr0, al0, qc.n_rows, ic.n_rows)
            log("config dense, heavy-dim part off: avg %.4f ms" % k0.mean())
        del qc, ic
    dense_ab = None
    if not args.no_dense_ab:
        k1, pr1, al1 = time_chunks(q_host, i_host, C, dense=True)
        k0, pr0, al0 = time_chunks(q_host, i_host, C, dense=False)
        dense_ab = {"on": summary(k1, pr1, al1, n_q, n_i), "off": summary(k0, pr0, al0, n_q, n_i),
                    "note": "same workload, prepared with the heavy-dim matrix-core part on "
                            "(default) and off (SPS_DENSE=0: every dim through the inverted "
                            "lists)"}
        log("%s heavy-dim part on/off: avg launch %.4f / %.4f ms" % (w.name, k1.mean(),
                                                                    k0.mean()))

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        o = oracle.default()
        hc = host_cpus()
        pin = hc["cores_used"]
        nthreads = len(pin)

        def oracle_rate(qh, ih, rows=None):
            qn, _ = o.row_norms(qh)
            inn, _ = o.row_norms(ih)
            t = time.perf_counter()
            o.scores(qh, ih, q_norm=qn, i_norm=inn, q_rows=rows, n_threads=nthreads,
                     pin_cpus=pin)
            dt = time.perf_counter() - t
            pairs = (qh.n_rows if rows is None else len(rows)) * float(ih.n_rows)
            return pairs / dt, dt, pairs

        full = {}
        for name in ("tiny", "mid"):
            qc, ic, _ = synth.make_workload(name)
            r, dt, pairs = oracle_rate(qc, ic)
            full[name] = {"scores_per_s": r, "seconds": dt, "pairs": pairs}
            del qc, ic
        rows = np.arange(min(args.cpu_rows, n_q))
        r, dt, pairs = oracle_rate(q_host, i_host, rows)
        cpu = {"value": r, "unit": "scores/s", "cores": nthreads, "kind": "oracle",
               "sample": "%d query rows x all %d items (%.3g pairs) of the %s workload, float64 "
                         "two-pointer merge, %.1f s wall" % (len(rows), n_i, pairs, w.name, dt),
               "threads_pinned": True, "cpu_model": hc["cpu_model"],
               "affinity_cores": hc["affinity_cores"], "cgroup_cpu_quota": hc["cgroup_cpu_quota"],
               "omp_num_threads": hc["omp_num_threads"],
               "full_runs": full,
               "extrapolated_whole_run_s": float(n_q) * n_i / r,
               "extrapolated_note": "EXTRAPOLATED, not measured: n_query x n_item / the sampled "
                                    "rate"}
        log("cpu oracle: %.3g scores/s on %d pinned threads (%s; mask %d cores); full tiny %.3g, "
            "mid %.3g scores/s; whole %s run extrapolated to %.0f s" % (
                r, nthreads, hc["cpu_model"], hc["affinity_cores"],
                full["tiny"]["scores_per_s"], full["mid"]["scores_per_s"], w.name,
                cpu["extrapolated_whole_run_s"]))

    res = {
        "metric": "cosine scores/sec + achieved HBM GB/s vs peak, 50k q x 2M items, nnz~43",
        "value": value,
        "unit": "scores/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 (light dims: fp32 products into int32 fixed point; heavy dims: split-fp16 "
                 "matrix cores, fp32 accumulation)",
        "data": "synthetic (seeded Philox CSR shaped like the page's workload)",
        "config": {"workload": "%s: %s" % (w.name, w.description), "n_query": n_q,
                   "n_item": n_i, "dim": w.dim, "chunk_size": C, "chunks": n_chunks,
                   "item_nnz": int(i_host.nnz), "query_nnz": int(q_host.nnz)},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic},
        "cpu_baseline": cpu,
        "breakdown_ms": {"prepare": prep_ms, "score_loop": loop_ms,
                         "score_launch_avg": avg_launch_ms,
                         "score_launch_median": float(np.median(main.launch_ms())),
                         "launches_timed": len(main.samples),
                         "step_median": median_step_ms},
        "step_hbm_gbps_algorithmic": float(alg_bytes.sum()) / (ms_per_step * 1e-3) / 1e9,
        "write_ceiling_gbps": write_ceiling,
        "frac_of_write_ceiling": achieved / write_ceiling,
        "variants": {"fp16": half, "threshold": thr, "host_stream": host, "bsc": bscv,
                     "configs": configs, "heavy_dims_on_off": dense_ab},
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
