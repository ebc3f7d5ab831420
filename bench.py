#!/usr/bin/env python3
"""Benchmark of the fused int8 IVF + Bloom-signature top-k search on one MI355X.

A step is one svt_search over one batch of synthetic queries: coarse probe, Bloom filter, int8 score
and top-k select, merged to the final top-k, all in the gfx950 kernels.  Inputs are resident in HBM
before the timed region starts.  The default workload is the 80M-item catalogue (d = 128, nlist =
16384, Zipf 0.8 cluster sizes, 128-bit signatures), nprobe 64, top-2048, query batches of 256.

Printed: one JSON line on stdout (progress goes to stderr) with
  value        eligible (query, item) pairs scored per second over the timed steps
  roofline     the scan kernel's algorithmic bytes per launch / its average duration (HIP events on the
               search stream over the timed region) against the 8 TB/s HBM peak
  cpu_baseline the CPU oracle timed on a bounded sample of the same workload on the host cores
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
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU-seconds of oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic", default=None, help="traffic summary (profiles/); default by workload")
    ap.add_argument("--print-sha", action="store_true", help="print the hash of the kernel sources and exit")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="run one device copy of this many MiB after the timed region (counter calibration)")
    return ap.parse_args()


def kernel_source_hash() -> str:
    """Hash of the code the scan kernel is built from (its source, the shared device helpers and the
    constants), with comments removed and whitespace collapsed, so that a comment edit keeps it."""
    h = hashlib.sha256()
    for f in ("svt_kernels.hip", "svt_device.h", "svt_internal.h"):
        with open(os.path.join(ROOT, "int8_ivf_ann_amd", "csrc", f)) as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def algorithmic_bytes(cat, sigs_sorted, offsets, queries, masks, nprobe, W, d):
    """Bytes the scan must move for one batch when every probed cluster is read once per batch:
    signatures of every item of the union of probed clusters, plus the row of every item eligible for
    at least one query probing its cluster.  Also returns the number of eligible (query, item) pairs."""
    C = cat.centroids.astype(np.float64)
    S = queries.astype(np.float64) @ C.T            # exact: |score| < 2^21
    nlist = C.shape[0]
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
            ok = np.all((sg & masks[b]) == masks[b], axis=1)
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
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}); "
              "the sharding design is described in DESIGN.md", file=sys.stderr)
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
        batches.append(dict(q=qs.queries, m=masks, q_d=torch.from_numpy(qs.queries).cuda(),
                            m_d=torch.from_numpy(masks.view(np.int64)).cuda()))
    ws = ix.workspace(B, nprobe, k)
    outs = dict(out_ids=torch.empty((B, k), dtype=torch.int64, device="cuda"),
                out_scores=torch.empty((B, k), dtype=torch.int32, device="cuda"),
                out_fscores=torch.empty((B, k), dtype=torch.float32, device="cuda"),
                out_counts=torch.empty((B,), dtype=torch.int32, device="cuda"))
    stats = [torch.empty((B, 2), dtype=torch.int64, device="cuda") for _ in batches]

    def step(i):
        bt = batches[i % len(batches)]
        svt.svt_search(ix.handle, bt["q_d"], bt["m_d"], nprobe, k, workspace=ws, out_stats=stats[i % len(batches)],
                       **outs)

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
    tpath = args.traffic or os.path.join(ROOT, "profiles", f"traffic_k_scan_{name}_b{B}.md")
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
        threads = max(1, min(16, os.cpu_count() or 1))
        bt = batches[0]
        # one query first, to size a sample of about args.cpu_seconds of CPU work
        ts = time.perf_counter()
        orc.search(cat.items, sigs, cat.list_of, cat.centroids, cat.item_scale, bt["q"][:1], bt["m"][:1], nprobe, k)
        one = time.perf_counter() - ts
        n_s = int(min(B, max(threads, round(args.cpu_seconds / max(one, 1e-6)))))
        ts = time.perf_counter()
        _, _, _, _, st = orc.search(cat.items, sigs, cat.list_of, cat.centroids, cat.item_scale, bt["q"][:n_s],
                                    bt["m"][:n_s], nprobe, k, n_threads=threads)
        cs = time.perf_counter() - ts
        cpu = {"value": float(st[:, 1].sum() / cs), "unit": "items/s", "cores": threads, "kind": "oracle",
               "sample": f"first {n_s} queries of batch 0 of the same workload ({int(st[:, 1].sum())} eligible pairs, "
                         f"{cs:.2f} s wall on {threads} threads)"}
        log(f"[bench] cpu oracle: {cpu['value']:.3e} items/s on {threads} threads ({n_s} queries, {cs:.2f}s)")

    wl = (f"{name}: {cat.n_items} items, d={d}, nlist={cfg['nlist']} "
          f"({'Zipf ' + str(cfg['cluster_zipf']) if cfg['cluster_zipf'] else 'uniform'} cluster sizes), "
          f"{64 * W}-bit Bloom signatures, nprobe={nprobe}, top-{k}, batch {B}")
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
                   "nlist": cfg["nlist"], "nprobe": nprobe, "k": k, "sig_bits": 64 * W},
        "qps": B * args.steps / elapsed,
        "items_scanned_per_s": steps_scanned / elapsed,
        "stage_ms_per_step": {kname: v / max(n_stage, 1) for kname, v in stage_ms.items()},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "kernel": "k_scan",
                     "algorithmic_bytes_per_launch": alg_per_launch},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    ix.close()


if __name__ == "__main__":
    main()
