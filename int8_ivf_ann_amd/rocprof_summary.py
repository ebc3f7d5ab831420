"""Short text summaries of rocprofv3 result databases (the rocpd SQLite files rocprofv3 writes).

    python -m int8_ivf_ann_amd.rocprof_summary kernels RESULTS.db [--match k_scan] [--command "..."]
        per-kernel dispatch count and duration statistics (microseconds)

    python -m int8_ivf_ann_amd.rocprof_summary counters RESULTS.db [RESULTS.db ...] --match k_scan [--command "..."]
        mean value per dispatch of every counter collected for the matching kernels (one line per counter)

    python -m int8_ivf_ann_amd.rocprof_summary traffic --fetch FETCH.db --write WRITE.db --kernel k_scan \
        --calib copyBuffer --calib-bytes 1073741824 --sha SHA [--command-fetch ...] [--command-write ...]
        HBM bytes per dispatch of a kernel from FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by
        what the same counter reads for a plain copy kernel of known size run in the same process

The summaries are Markdown text; ``traffic`` ends with ``key: value`` lines that bench.py reads
(``hbm_bytes_per_launch``, ``kernel_source_sha``).
"""
from __future__ import annotations

import argparse
import sqlite3
import statistics
import sys
from typing import Dict, List, Optional


def _kernels(db: str):
    con = sqlite3.connect(db)
    rows = con.execute("select name, duration from kernels").fetchall()
    con.close()
    out: Dict[str, List[float]] = {}
    for name, dur in rows:
        out.setdefault(name, []).append(dur / 1000.0)   # ns -> us
    return out


def _counter(db: str, counter: str):
    con = sqlite3.connect(db)
    rows = con.execute("select kernel_name, value from counters_collection where counter_name = ?",
                       (counter,)).fetchall()
    con.close()
    out: Dict[str, List[float]] = {}
    for name, v in rows:
        out.setdefault(name, []).append(float(v))
    return out


def kernels_md(db: str, match: Optional[List[str]], command: Optional[str]) -> str:
    ks = _kernels(db)
    lines = []
    if command:
        lines += ["command:", "", "    " + command, ""]
    lines += ["| kernel | dispatches | avg us | min us | max us | total us |", "|---|---|---|---|---|---|"]
    for name, d in sorted(ks.items(), key=lambda kv: -sum(kv[1])):
        if match and not any(m in name for m in match):
            continue
        lines.append(f"| `{name[:90]}` | {len(d)} | {statistics.mean(d):.2f} | {min(d):.2f} | {max(d):.2f} | "
                     f"{sum(d):.1f} |")
    return "\n".join(lines) + "\n"


def counters_md(dbs: List[str], match: str, commands: Optional[List[str]]) -> str:
    lines = []
    for c in commands or []:
        lines += ["    " + c, ""]
    lines += ["| kernel | counter | dispatches | mean per dispatch |", "|---|---|---|---|"]
    for db in dbs:
        con = sqlite3.connect(db)
        rows = con.execute("select kernel_name, counter_name, value from counters_collection").fetchall()
        con.close()
        acc: Dict[tuple, List[float]] = {}
        for name, cn, v in rows:
            if match in name:
                acc.setdefault((name, cn), []).append(float(v))
        for (name, cn), v in sorted(acc.items()):
            lines.append(f"| `{name[:40]}` | {cn} | {len(v)} | {statistics.mean(v):.6g} |")
    return "\n".join(lines) + "\n"


def _one(d: Dict[str, List[float]], sub: str, what: str) -> List[float]:
    hits = [v for k, v in d.items() if sub in k]
    if len(hits) != 1:
        raise SystemExit(f"{what}: {len(hits)} kernels match {sub!r}: {[k for k in d if sub in k]}")
    return hits[0]


def traffic_md(fetch_db: str, write_db: str, kernel: str, calib: str, calib_bytes: int, sha: str,
               cmd_fetch: Optional[str], cmd_write: Optional[str]) -> str:
    f = _counter(fetch_db, "FETCH_SIZE")
    w = _counter(write_db, "WRITE_SIZE")
    kf, kw = _one(f, kernel, "FETCH_SIZE"), _one(w, kernel, "WRITE_SIZE")
    # the copy dispatch of the calibration is the largest dispatch of the copy kernel
    cf, cw = max(_one(f, calib, "FETCH_SIZE")), max(_one(w, calib, "WRITE_SIZE"))
    f_scale = calib_bytes / (cf * 1024.0)
    w_scale = calib_bytes / (cw * 1024.0)
    rd = statistics.mean(kf) * 1024.0 * f_scale
    wr = statistics.mean(kw) * 1024.0 * w_scale
    lines = []
    if cmd_fetch:
        lines += ["FETCH_SIZE pass:", "", "    " + cmd_fetch, ""]
    if cmd_write:
        lines += ["WRITE_SIZE pass:", "", "    " + cmd_write, ""]
    lines += [
        f"calibration: a plain device copy of {calib_bytes} bytes reads FETCH_SIZE {cf:.1f} KiB and WRITE_SIZE "
        f"{cw:.1f} KiB, so FETCH_SIZE is scaled by {f_scale:.4f} and WRITE_SIZE by {w_scale:.4f}",
        "",
        f"| kernel | dispatches | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | read bytes | write bytes |",
        "|---|---|---|---|---|---|",
        f"| `{kernel}` | {len(kf)} | {statistics.mean(kf):.1f} | {statistics.mean(kw):.1f} | {rd:.4g} | {wr:.4g} |",
        "",
        f"hbm_read_bytes_per_launch: {rd:.0f}",
        f"hbm_write_bytes_per_launch: {wr:.0f}",
        f"hbm_bytes_per_launch: {rd + wr:.0f}",
        f"kernel_source_sha: {sha}",
    ]
    return "\n".join(lines) + "\n"


def read_traffic(path: str) -> Dict[str, str]:
    """``key: value`` lines of a traffic summary."""
    import re
    out = {}
    with open(path) as fh:
        for line in fh:
            m = re.match(r"^([a-z_]+): (\S+)\s*$", line)
            if m:
                out[m.group(1)] = m.group(2)
    return out


def main(argv=None) -> None:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    k = sub.add_parser("kernels")
    k.add_argument("db")
    k.add_argument("--match", action="append")
    k.add_argument("--command")
    c = sub.add_parser("counters")
    c.add_argument("dbs", nargs="+")
    c.add_argument("--match", required=True)
    c.add_argument("--command", action="append")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--calib", default="copyBuffer")
    t.add_argument("--calib-bytes", type=int, required=True)
    t.add_argument("--sha", required=True)
    t.add_argument("--command-fetch")
    t.add_argument("--command-write")
    a = ap.parse_args(argv)
    if a.cmd == "kernels":
        sys.stdout.write(kernels_md(a.db, a.match, a.command))
    elif a.cmd == "counters":
        sys.stdout.write(counters_md(a.dbs, a.match, a.command))
    else:
        sys.stdout.write(traffic_md(a.fetch, a.write, a.kernel, a.calib, a.calib_bytes, a.sha, a.command_fetch,
                                    a.command_write))


if __name__ == "__main__":
    main()
