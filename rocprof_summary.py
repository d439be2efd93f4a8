"""Condense rocprofv3 CSV output into the short text summaries kept in profiles/.

  python rocprof_summary.py trace DIR --out FILE --command CMD
  python rocprof_summary.py counters --workload NAME \
      --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR \
      --copy-bytes N --out FILE --command CMD [--kernel decode_attn_stream_kernel]
  python rocprof_summary.py pmc DIR --kernel PREFIX --out FILE --command CMD

`trace` keeps the per-kernel statistics of a `--kernel-trace --stats` run.
`counters` turns FETCH_SIZE / WRITE_SIZE (KiB per dispatch) into HBM bytes
per launch of the attention kernel (or, for a decode-projection workload,
of gemm_m1_kernel): each counter is scaled by the ratio of
known bytes to the same counter's reading for a plain copy kernel
(`bench.py --copy-only N`, which reads N and writes N bytes per launch).
The summary records the hash of the kernel sources it was taken on;
bench.py reports the traffic only while that hash still matches.
`pmc` tabulates the median per dispatch of every counter a `--pmc` run
collected for the kernels whose name starts with PREFIX.
"""
from __future__ import annotations

import argparse
import csv
import glob
import os
import statistics
import sys


def _find(directory: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    return hits[0]


def _counter_values(directory: str, counter: str, kernel_prefix: str):
    rows = csv.DictReader(open(_find(directory, "counter_collection.csv")))
    vals = [float(r["Counter_Value"]) for r in rows
            if r["Counter_Name"] == counter and r["Kernel_Name"].startswith(kernel_prefix)]
    if not vals:
        raise ValueError(f"no {counter} rows for {kernel_prefix} in {directory}")
    return vals


def trace(args):
    path = _find(args.dir, "kernel_stats.csv")
    rows = list(csv.DictReader(open(path)))
    lines = [f"# rocprofv3 kernel statistics ({os.path.basename(path)})",
             f"# command: {args.command}",
             f"{'kernel':40s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} "
             f"{'max_us':>10s} {'pct':>7s}"]
    for r in rows:
        lines.append(f"{r['Name'][:40]:40s} {int(r['Calls']):6d} "
                     f"{float(r['AverageNs']) / 1e3:10.3f} {float(r['MinNs']) / 1e3:10.3f} "
                     f"{float(r['MaxNs']) / 1e3:10.3f} {float(r['Percentage']):7.2f}")
    text = "\n".join(lines) + "\n"
    _write(args.out, text)


def counters(args):
    from bench import (GEMM_SOURCES, attention_algorithmic_bytes, gemm_algorithmic_bytes,
                       kernel_source_hash, step_fuses_append)
    from workloads import CONFIGS, GEMM_CONFIGS, Workload
    kib = 1024.0
    copy_prefix = "vectorized_elementwise_kernel"
    # the copy run's first elementwise launch converts the source (fp32 ->
    # fp16, reads twice the bytes); the copies proper are the rest
    cf = _counter_values(args.copy_fetch, "FETCH_SIZE", copy_prefix)[1:]
    cw = _counter_values(args.copy_write, "WRITE_SIZE", copy_prefix)[1:]
    f_fetch = args.copy_bytes / (statistics.median(cf) * kib)
    f_write = args.copy_bytes / (statistics.median(cw) * kib)
    af = _counter_values(args.fetch, "FETCH_SIZE", args.kernel)
    aw = _counter_values(args.write, "WRITE_SIZE", args.kernel)
    fetch_b = statistics.median(af) * kib * f_fetch
    write_b = statistics.median(aw) * kib * f_write
    if args.workload in GEMM_CONFIGS:
        alg = gemm_algorithmic_bytes(GEMM_CONFIGS[args.workload])
        src_hash = kernel_source_hash(GEMM_SOURCES)
    else:
        w = Workload(CONFIGS[args.workload])
        # the kernel's own bytes: the appended rows only when it does the append
        alg = attention_algorithmic_bytes(w, with_append=step_fuses_append(w))
        src_hash = kernel_source_hash()
    lines = [
        f"# HBM traffic of {args.kernel} on workload {args.workload}",
        f"# command: {args.command}",
        f"kernel: {args.kernel}",
        f"workload: {args.workload}",
        f"kernel_source_sha256_16: {src_hash}",
        f"dispatches_fetch: {len(af)}",
        f"dispatches_write: {len(aw)}",
        f"fetch_size_kib_median: {statistics.median(af):.3f}",
        f"write_size_kib_median: {statistics.median(aw):.3f}",
        f"copy_bytes_per_launch: {args.copy_bytes}",
        f"copy_fetch_size_kib_median: {statistics.median(cf):.3f}",
        f"copy_write_size_kib_median: {statistics.median(cw):.3f}",
        f"fetch_scale: {f_fetch:.4f}",
        f"write_scale: {f_write:.4f}",
        f"hbm_read_bytes_per_launch: {fetch_b:.0f}",
        f"hbm_write_bytes_per_launch: {write_b:.0f}",
        f"hbm_bytes_per_launch: {fetch_b + write_b:.0f}",
        f"algorithmic_bytes_per_launch: {alg}",
        f"traffic_over_algorithmic: {(fetch_b + write_b) / alg:.4f}",
    ]
    _write(args.out, "\n".join(lines) + "\n")


def pmc(args):
    rows = [r for r in csv.DictReader(open(_find(args.dir, "counter_collection.csv")))
            if r["Kernel_Name"].startswith(args.kernel)]
    if not rows:
        raise ValueError(f"no rows for {args.kernel} in {args.dir}")
    by = {}
    for r in rows:
        by.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    lines = [f"# rocprofv3 counters of {args.kernel}* (median per dispatch)",
             f"# command: {args.command}",
             f"{'counter':32s} {'dispatches':>10s} {'median':>16s}"]
    for name in sorted(by):
        lines.append(f"{name:32s} {len(by[name]):10d} {statistics.median(by[name]):16.1f}")
    _write(args.out, "\n".join(lines) + "\n")


def _write(path, text):
    if path == "-":
        sys.stdout.write(text)
        return
    with open(path, "w") as f:
        f.write(text)
    sys.stdout.write(text)


def main(argv=None):
    root = os.path.dirname(os.path.abspath(__file__))
    sys.path.insert(0, root)
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--out", default="-")
    t.add_argument("--command", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--workload", required=True)
    c.add_argument("--kernel", default="decode_attn_stream_kernel")
    for k in ("fetch", "write", "copy_fetch", "copy_write"):
        c.add_argument("--" + k.replace("_", "-"), dest=k, required=True)
    c.add_argument("--copy-bytes", type=int, required=True)
    c.add_argument("--out", default="-")
    c.add_argument("--command", required=True)
    m = sub.add_parser("pmc")
    m.add_argument("dir")
    m.add_argument("--kernel", required=True)
    m.add_argument("--out", default="-")
    m.add_argument("--command", required=True)
    args = ap.parse_args(argv)
    {"trace": trace, "counters": counters, "pmc": pmc}[args.cmd](args)


if __name__ == "__main__":
    main()
