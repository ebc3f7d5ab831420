#!/usr/bin/env python3
"""Benchmark of the fused int8 IVF + Bloom-signature top-k search on one MI355X.

A step is one svt_search over one batch of synthetic queries: coarse probe, Bloom filter, int8 score
and top-k select, merged to the final top-k, all in the gfx950 kernels.  Inputs are resident in HBM
before the timed region starts.  The default workload is the 80M-item catalogue (d = 128, nlist =
16384, Zipf 0.8 cluster sizes, 128-bit signatures), nprobe 64, top-2048, query batches of 256.

Printed: one JSON line on stdout (progress goes to stderr) with
  value        eligible (query, item) pairs scored per second over the timed steps
  roofline     the scan kernel of the path taken (k_scan, k_tscan or k_xscan): algorithmic bytes per launch
               / its average duration (HIP events on the search stream over the timed region) against the
               8 TB/s HBM peak; also the same bytes per whole step (step_frac), the streaming-read rate
               measured in the same run (read_ceiling) and the fabric traffic of the last counter run
               taken on the current sources (traffic, else null)
  cpu_baseline the CPU oracle timed on bounded samples of the same workload, on up to 16 host threads and
               on one thread, with the host's thread count and CPU model
  latency      (batch 1 by default) p50 / p99 of single searches over 1000 distinct queries
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "eligible items scored/sec (int8 IVF+Bloom, top-2048); achieved HBM GB/s %"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="80m", help="preset: tiny, 1m, 10m, 80m, exh")
    ap.add_argument("--batch", type=int, default=None, help="queries per step (default: preset's largest)")
    ap.add_argument("--batches", type=int, default=4, help="distinct query batches cycled over the steps")
    ap.add_argument("--path", default="auto", choices=["auto", "query", "tile", "large_k"], help="search path")
    ap.add_argument("--k", type=int, default=None, help="top-k (default: the preset's; above 2048: large-k path)")
    ap.add_argument("--mask-groups", type=int, default=1,
                    help="request masks per query (an item is eligible when any passes); group 0 is the query's own "
                         "required tokens, group g those of another synthetic query")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU-seconds of oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic", default=None, help="traffic summary (profiles/); default by workload")
    ap.add_argument("--print-sha", action="store_true", help="print the hash of the kernel sources and exit")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="run one device copy of this many MiB after the timed region (counter calibration)")
    ap.add_argument("--latency-queries", type=int, default=None,
                    help="searches timed one by one for latency percentiles (default: 1000 at batch 1, else 0)")
    ap.add_argument("--no-read-ceiling", action="store_true", help="skip the streaming-read probe")
    ap.add_argument("--no-rerank", action="store_true", help="skip the rerank measurement")
    ap.add_argument("--rerank-k", type=int, default=256, help="rerank: candidates kept per query")
    return ap.parse_args()


def kernel_source_hash() -> str:
    """Hash of everything the search kernels are built from: every source of the library (kernels, device
    helpers, constants, the host code that sets launch shapes and paths) with comments removed and
    whitespace collapsed, so that a comment edit keeps it, plus the compiler flags."""
    from int8_ivf_ann_amd import build
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "int8_ivf_ann_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if not f.endswith((".hip", ".h", ".cpp")):
            continue
        with open(os.path.join(csrc, f)) as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(f.encode() + b"\0" + " ".join(src.split()).encode())
    h.update(" ".join(build.COMMON[:4] + build.DEVICE_FLAGS + [build.ARCH]).encode())
    return h.hexdigest()[:16]


def read_ceiling_gbs(torch, gib: int = 4, reps: int = 5) -> float:
    """Streaming-read rate of this GPU: torch's sum over a gib-GiB int64 tensor, best of reps."""
    x = torch.ones((gib << 30) // 8, dtype=torch.int64, device="cuda")
    best = 0.0
    for _ in range(reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        s = x.sum()
        e1.record()
        e1.synchronize()
        best = max(best, x.numel() * 8 / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del x, s
    return best


FP32_MATRIX_PEAK_TFLOPS = 157.3   # MI355X dense float32 matrix rate
RERANK_EXPERTS, RERANK_HIDDEN = 4, 16


def rerank_leg(args, torch, svt, ix, cat, bt, cand, d):
    """Times svt_rerank over one batch's search results (the candidates) with a seeded random net;
    the first layer (2 E H d flops per candidate) runs on the float32 matrix cores."""
    import synth
    rng = np.random.default_rng(2024)
    net = synth.rerank_net(rng, d, RERANK_EXPERTS, RERANK_HIDDEN)
    tnet = {key: torch.from_numpy(v).cuda() for key, v in net.items()}
    B, n_cand = cand.shape
    k_out = args.rerank_k
    outs = dict(out_ids=torch.empty((B, k_out), dtype=torch.int64, device="cuda"),
                out_scores=torch.empty((B, k_out), dtype=torch.float32, device="cuda"),
                out_counts=torch.empty((B,), dtype=torch.int32, device="cuda"))
    for _ in range(3):
        ix.rerank(bt["q_d"], cand, tnet, k_out, **outs)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()   # on torch's current stream, the one the binding launches on
    for _ in range(args.steps):
        ix.rerank(bt["q_d"], cand, tnet, k_out, **outs)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    cand_h = cand.cpu().numpy()
    n_valid = int((cand_h >= 0).sum())
    U = RERANK_EXPERTS * RERANK_HIDDEN
    flops = n_valid * 2.0 * U * d + B * 2.0 * RERANK_EXPERTS * d
    achieved = flops / (ms * 1e-3) / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import rerank as R
        n_s = min(B, 16)
        t0 = time.perf_counter()
        R.rerank(cat.items, cat.item_scale, bt["q"][:n_s], None, cand_h[:n_s], net, k_out)
        cs = time.perf_counter() - t0
        nv_s = int((cand_h[:n_s] >= 0).sum())
        cpu = {"value": nv_s / cs, "unit": "candidates/s", "cores": 1, "kind": "oracle",
               "sample": f"first {n_s} queries of the batch ({nv_s} candidates, {cs:.2f} s, numpy float64)"}
    traffic = None   # fabric bytes per launch from the committed summary, when taken on these sources
    tpath = os.path.join(ROOT, "profiles", f"traffic_k_rerank_{args.workload}_b{B}.md")
    if os.path.exists(tpath):
        from int8_ivf_ann_amd.rocprof_summary import read_traffic
        tj = read_traffic(tpath)
        if tj.get("kernel_source_sha") == kernel_source_hash():
            traffic = float(tj["hbm_bytes_per_launch"])
    res = {"kernel": "k_rerank", "candidates_per_s": n_valid / (ms * 1e-3), "ms_per_launch": ms,
           "config": {"batch": B, "n_cand": n_cand, "k_out": k_out, "experts": RERANK_EXPERTS,
                      "hidden": RERANK_HIDDEN, "dim": d, "candidates": "the search's top-k of the same batch"},
           "roofline": {"bound": "mfma", "achieved": achieved, "peak": FP32_MATRIX_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": achieved / FP32_MATRIX_PEAK_TFLOPS, "flops_per_launch": flops,
                        "traffic": traffic},
           "cpu_baseline": cpu}
    log(f"[bench] rerank {B}x{n_cand} -> {k_out}: {ms:.4f} ms/launch, {achieved:.1f} TFLOP/s "
        f"({100 * achieved / FP32_MATRIX_PEAK_TFLOPS:.1f}% of fp32 matrix peak)")
    return res


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def algorithmic_bytes(cat, sigs_sorted, offsets, queries, masks, nprobe, W, d):
    """Bytes the scan must move for one batch when every probed cluster is read once per batch:
    signatures of every item of the union of probed clusters, plus the row of every item eligible for
    at least one query probing its cluster.  Also returns the number of eligible (query, item) pairs.
    masks: [B, W] or [B, G, W] (eligible when any group passes)."""
    nlist = cat.centroids.shape[0]
    if masks.ndim == 2:
        masks = masks[:, None, :]

    def passes(sg, mb):   # items of sg passing any of the masks mb [G, W]
        ok = np.zeros(sg.shape[0], bool)
        for m in mb:
            ok |= np.all((sg & m) == m, axis=1)
        return ok

    if nprobe == nlist:
        # every query probes every cluster: one pass over the catalogue per query
        need = np.zeros(sigs_sorted.shape[0], bool)
        pairs = 0
        for b in range(queries.shape[0]):
            ok = passes(sigs_sorted, masks[b])
            pairs += int(ok.sum())
            need |= ok
            if b % 8 == 7:
                log(f"[bench] bookkeeping: {b + 1} of {queries.shape[0]} queries")
        sig_bytes = sigs_sorted.shape[0] * 8 * W
        rows = int(need.sum())
        return sig_bytes + rows * d, sig_bytes, rows * d, pairs, nlist
    C = cat.centroids.astype(np.float64)
    S = queries.astype(np.float64) @ C.T            # exact: |score| < 2^21
    cl_q = {}
    for b in range(queries.shape[0]):
        s = S[b]
        order = np.lexsort((np.arange(nlist), -s))[:nprobe]
        for c in order.tolist():
            cl_q.setdefault(c, []).append(b)
    sig_bytes = 0
    rows = 0
    pairs = 0
    for c, qs in cl_q.items():
        a, e = int(offsets[c]), int(offsets[c + 1])
        if e == a:
            continue
        sg = sigs_sorted[a:e]
        need = np.zeros(e - a, bool)
        for b in qs:
            ok = passes(sg, masks[b])
            pairs += int(ok.sum())
            need |= ok
        sig_bytes += (e - a) * 8 * W
        rows += int(need.sum())
    return sig_bytes + rows * d, sig_bytes, rows * d, pairs, len(cl_q)


def main():
    args = parse()
    if args.print_sha:
        print(kernel_source_hash())
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}); "
              "an index would shard by cluster ranges, each GPU scanning its own clusters for every query "
              "and the per-GPU top-k lists merged afterwards", file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    from int8_ivf_ann_amd import svt

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    name = args.workload
    t0 = time.time()
    cat = synth.catalogue(name)
    cfg = cat.cfg
    W, h, d, nprobe, k = cfg["sig_words"], cfg["n_hashes"], cfg["dim"], cfg["nprobe"], cfg["k"]
    B = args.batch or max(cfg["batches"])
    if args.k is not None:
        k = args.k
    log(f"[bench] generated {name}: {cat.n_items} items d={d} nlist={cfg['nlist']} in {time.time() - t0:.1f}s")
    t0 = time.time()
    sigs = svt.svt_bloom_sign(cat.tokens, h, W)
    cat.tokens = None
    ix = svt.Index(cat.items, sigs, cat.list_of, cat.centroids, cat.item_scale)
    log(f"[bench] signed + uploaded in {time.time() - t0:.1f}s")

    # distinct query batches, resident on the device
    batches = []
    for i in range(args.batches):
        qs = synth.queries(cat, B, offset=i * B)
        masks = np.stack([svt.svt_bloom_mask(qs.required(b), h, W) for b in range(B)])
        if args.mask_groups > 1:
            groups = [masks]
            for g in range(1, args.mask_groups):
                alt = synth.queries(cat, B, offset=(args.batches * g + i) * B)
                groups.append(np.stack([svt.svt_bloom_mask(alt.required(b), h, W) for b in range(B)]))
            masks = np.ascontiguousarray(np.stack(groups, axis=1))   # [B, G, W]
        batches.append(dict(q=qs.queries, m=masks, q_d=torch.from_numpy(qs.queries).cuda(),
                            m_d=torch.from_numpy(masks.view(np.int64)).cuda()))
    opts = svt.make_options(args.path, mask_groups=args.mask_groups)
    path = svt.svt_search_path(ix.handle, B, nprobe, k, opts)
    kernel = {"query": "k_scan", "tile": "k_tscan", "exhaustive": "k_xscan", "large_k": "k_lk_scan"}[path]
    ws = ix.workspace(B, nprobe, k, opts)
    log(f"[bench] workspace {ws.numel() / 2**20:.1f} MiB (path {args.path}: {path}, scan kernel {kernel})")
    outs = dict(out_ids=torch.empty((B, k), dtype=torch.int64, device="cuda"),
                out_scores=torch.empty((B, k), dtype=torch.int32, device="cuda"),
                out_fscores=torch.empty((B, k), dtype=torch.float32, device="cuda"),
                out_counts=torch.empty((B,), dtype=torch.int32, device="cuda"))
    stats = [torch.empty((B, 2), dtype=torch.int64, device="cuda") for _ in batches]

    def step(i):
        bt = batches[i % len(batches)]
        svt.svt_search(ix.handle, bt["q_d"], bt["m_d"], nprobe, k, workspace=ws, out_stats=stats[i % len(batches)],
                       opts=opts, **outs)

    for i in range(max(args.warmup, len(batches))):
        step(i)
    torch.cuda.synchronize()
    elig = [int(s[:, 1].sum().item()) for s in stats]
    scanned = [int(s[:, 0].sum().item()) for s in stats]

    # timed region: K steps; HIP events on the search stream around the scan kernel only (two event
    # records per step), for the scan's average launch duration
    svt.svt_profile_read()               # drop anything recorded before
    svt.svt_profile_enable(2)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    svt.svt_profile_enable(False)
    scan_prof, n_prof = svt.svt_profile_read()
    elapsed = t1 - t0
    steps_elig = sum(elig[i % len(batches)] for i in range(args.steps))
    steps_scanned = sum(scanned[i % len(batches)] for i in range(args.steps))
    value = steps_elig / elapsed
    # stage breakdown in a separate pass (an event around every stage), outside the timed region
    svt.svt_profile_enable(True)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    svt.svt_profile_enable(False)
    stage_ms, n_stage = svt.svt_profile_read()
    log(f"[bench] {args.steps} steps in {elapsed * 1e3:.2f} ms; stages of a separate profiled pass (ms/step): "
        + ", ".join(f"{kname} {v / max(n_stage, 1):.4f}" for kname, v in stage_ms.items()))

    # latency: searches of one batch timed one by one (distinct queries), host wall clock around the
    # search and a synchronisation, and HIP events on the search stream
    lat = None
    n_lat = args.latency_queries if args.latency_queries is not None else (1000 if B == 1 else 0)
    if n_lat > 0:
        ql = synth.queries(cat, n_lat * B, offset=args.batches * B)
        ml = np.stack([svt.svt_bloom_mask(ql.required(b), h, W) for b in range(n_lat * B)])
        ql_d = torch.from_numpy(ql.queries).cuda()
        ml_d = torch.from_numpy(ml.view(np.int64)).cuda()
        st_l = torch.empty((B, 2), dtype=torch.int64, device="cuda")
        host_ms, dev_ms, evs = [], [], []
        for i in range(n_lat + 5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            ts = time.perf_counter()
            e0.record()
            svt.svt_search(ix.handle, ql_d[(i % n_lat) * B:(i % n_lat + 1) * B], ml_d[(i % n_lat) * B:(i % n_lat + 1) * B],
                           nprobe, k, workspace=ws, out_stats=st_l, opts=svt.make_options(args.path), **outs)
            e1.record()
            torch.cuda.synchronize()
            if i >= 5:   # the first searches of new queries warm the caches
                host_ms.append((time.perf_counter() - ts) * 1e3)
                evs.append((e0, e1))
        dev_ms = [a.elapsed_time(b) for a, b in evs]
        pct = lambda v, p: float(np.percentile(np.asarray(v), p))
        lat = {"searches": n_lat, "batch": B,
               "host_ms": {"p50": pct(host_ms, 50), "p99": pct(host_ms, 99), "mean": float(np.mean(host_ms))},
               "device_ms": {"p50": pct(dev_ms, 50), "p99": pct(dev_ms, 99), "mean": float(np.mean(dev_ms))},
               "note": "host: wall clock of the search call plus a stream synchronisation; device: HIP events "
                       "recorded on the search stream before and after the search"}
        log(f"[bench] latency over {n_lat} searches of batch {B}: host p50 {lat['host_ms']['p50']:.4f} ms "
            f"p99 {lat['host_ms']['p99']:.4f} ms; device p50 {lat['device_ms']['p50']:.4f} ms "
            f"p99 {lat['device_ms']['p99']:.4f} ms")
        del ql_d, ml_d

    rerank = None
    if not args.no_rerank:
        bt = batches[0]
        cand = torch.empty((B, k), dtype=torch.int64, device="cuda")
        svt.svt_search(ix.handle, bt["q_d"], bt["m_d"], nprobe, k, workspace=ws, opts=opts,
                       **dict(outs, out_ids=cand))
        rerank = rerank_leg(args, torch, svt, ix, cat, bt, cand, d)
        del cand

    ceiling = None
    if not args.no_read_ceiling:
        ceiling = read_ceiling_gbs(torch)
        log(f"[bench] streaming-read ceiling (torch sum over 4 GiB): {ceiling:.1f} GB/s")

    if args.copy_calibration_mb > 0:
        # a plain copy of known size, for scaling hardware byte counters (read + write of n bytes each)
        nb = args.copy_calibration_mb << 20
        src = torch.ones(nb // 8, dtype=torch.int64, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy: {nb} bytes read, {nb} bytes written")
        del src, dst

    # algorithmic bytes of the scan kernel (numpy bookkeeping, outside the timed region)
    order = np.argsort(cat.list_of, kind="stable")
    offsets = np.zeros(cfg["nlist"] + 1, np.int64)
    np.cumsum(np.bincount(cat.list_of, minlength=cfg["nlist"]), out=offsets[1:])
    sigs_sorted = sigs[order]
    del order
    alg = [algorithmic_bytes(cat, sigs_sorted, offsets, bt["q"], bt["m"], nprobe, W, d) for bt in batches]
    del sigs_sorted
    for a, e in zip(alg, elig):
        assert a[3] == e, f"eligible pair count: bookkeeping {a[3]} vs kernel {e}"
    steps_alg = sum(alg[i % len(batches)][0] for i in range(args.steps))
    scan_ms = scan_prof["scan"] / max(n_prof, 1)   # timed region
    alg_per_launch = steps_alg / args.steps
    achieved = alg_per_launch / (scan_ms * 1e-3) / 1e9
    log(f"[bench] scan kernel: {alg_per_launch / 1e9:.3f} GB algorithmic per launch (sigs "
        f"{np.mean([a[1] for a in alg]) / 1e9:.3f} GB, rows {np.mean([a[2] for a in alg]) / 1e9:.3f} GB, "
        f"{np.mean([a[4] for a in alg]):.0f} distinct clusters) in {scan_ms:.4f} ms -> {achieved:.1f} GB/s")

    traffic = None
    tpath = args.traffic or os.path.join(ROOT, "profiles", f"traffic_{kernel}_{name}_b{B}.md")
    if os.path.exists(tpath):
        from int8_ivf_ann_amd.rocprof_summary import read_traffic
        tj = read_traffic(tpath)
        if tj.get("kernel_source_sha") == kernel_source_hash():
            traffic = float(tj["hbm_bytes_per_launch"])
        else:
            log(f"[bench] {tpath} was taken on other kernel sources: traffic reported as null")

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.Oracle()
        nproc = os.cpu_count() or 1
        threads = max(1, min(16, nproc))   # the GPU's share of the host: at most 16 threads
        bt = batches[0]
        # one query first, to size samples of about args.cpu_seconds of work on all threads and a third of
        # that on one thread
        ts = time.perf_counter()
        orc.search(cat.items, sigs, cat.list_of, cat.centroids, cat.item_scale, bt["q"][:1], bt["m"][:1], nprobe, k,
                   n_threads=1)
        one = time.perf_counter() - ts

        def run(n_q, n_thr):
            ts = time.perf_counter()
            _, _, _, _, st = orc.search(cat.items, sigs, cat.list_of, cat.centroids, cat.item_scale, bt["q"][:n_q],
                                        bt["m"][:n_q], nprobe, k, n_threads=n_thr)
            return int(st[:, 1].sum()), time.perf_counter() - ts

        n_1 = int(min(B, max(1, round(args.cpu_seconds / 3 / max(one, 1e-6)))))
        e1, c1 = run(n_1, 1)
        n_s = int(min(B, max(threads, round(args.cpu_seconds * threads / max(one, 1e-6)))))
        e_s, cs = run(n_s, threads)
        cpu = {"value": float(e_s / cs), "unit": "items/s", "cores": threads, "threads": threads, "kind": "oracle",
               "sample": f"first {n_s} queries of batch 0 of the same workload ({e_s} eligible pairs, "
                         f"{cs:.2f} s wall on {threads} threads)",
               "nproc": nproc, "cpu_model": cpu_model(),
               "single_thread": {"value": float(e1 / c1), "unit": "items/s", "threads": 1,
                                 "sample": f"first {n_1} queries of batch 0 ({e1} eligible pairs, {c1:.2f} s wall)"}}
        log(f"[bench] cpu oracle: {cpu['value']:.3e} items/s on {threads} threads ({n_s} queries, {cs:.2f}s); "
            f"{e1 / c1:.3e} items/s on 1 thread ({n_1} queries, {c1:.2f}s); nproc {nproc}, {cpu['cpu_model']}")

    wl = (f"{name}: {cat.n_items} items, d={d}, nlist={cfg['nlist']} "
          f"({'Zipf ' + str(cfg['cluster_zipf']) if cfg['cluster_zipf'] else 'uniform'} cluster sizes), "
          f"{64 * W}-bit Bloom signatures, nprobe={nprobe}, top-{k}, batch {B}"
          + (f", {args.mask_groups} masks per query (any passes)" if args.mask_groups > 1 else ""))
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "items/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic (seeded generator; inputs resident in HBM)",
        "config": {"workload": wl, "preset": name, "batch": B, "n_items": cat.n_items, "dim": d,
                   "nlist": cfg["nlist"], "nprobe": nprobe, "k": k, "sig_bits": 64 * W,
                   "mask_groups": args.mask_groups},
        "qps": B * args.steps / elapsed,
        "items_scanned_per_s": steps_scanned / elapsed,
        "stage_ms_per_step": {kname: v / max(n_stage, 1) for kname, v in stage_ms.items()},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "traffic_kind": "fabric bytes per launch: FETCH_SIZE + WRITE_SIZE (L2-to-fabric requests, "
                                     "Infinity Cache hits included), each scaled by the same counter over a "
                                     "device copy of known size",
                     "kernel": kernel, "path": path,
                     "algorithmic_bytes_per_launch": alg_per_launch,
                     "scan_ms": scan_ms,
                     "scan_stage": ("the large-k path's passes: every digit-count pass and pick, the collect pass and "
                                    "the sort (the algorithmic bytes are those of one pass)") if path == "large_k"
                                   else "the scan kernel",
                     "step_achieved": alg_per_launch / (elapsed / args.steps) / 1e9,
                     "step_frac": alg_per_launch / (elapsed / args.steps) / 1e9 / HBM_PEAK_GBS,
                     "read_ceiling": ceiling,
                     "frac_of_read_ceiling": (achieved / ceiling) if ceiling else None},
        "cpu_baseline": cpu,
    }
    if lat is not None:
        line["latency"] = lat
    if rerank is not None:
        line["rerank"] = rerank
    print(json.dumps(line), flush=True)
    ix.close()


if __name__ == "__main__":
    main()
