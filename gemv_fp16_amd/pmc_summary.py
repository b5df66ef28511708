"""Summaries of rocprofv3 counter runs (the *_counter_collection.csv files).

    python -m gemv_fp16_amd.pmc_summary table CSV [CSV ...]
        per kernel: dispatches and the mean value per dispatch of every counter
    python -m gemv_fp16_amd.pmc_summary trace KERNEL_TRACE_CSV [--kernel SUBSTRING]
        [--first N] [--skip N]
        durations of the kernels of a rocprofv3 --kernel-trace run: per kernel
        calls, mean / median / min / max in microseconds; with --kernel, the
        launches of the matching kernel(s) in dispatch order, optionally only
        launches skip .. skip + first - 1 of them, and each launch's duration
    python -m gemv_fp16_amd.pmc_summary traffic --fetch CSV --write CSV \
        --calib-fetch CSV --calib-write CSV --kernel SUBSTRING --key NAME \
        --algorithmic BYTES --command TEXT
        HBM bytes per launch of one kernel: FETCH_SIZE and WRITE_SIZE (KiB
        per dispatch), each scaled by what the same counter reads for the
        512 MiB device copy of profile_run.py's "copy" op against the bytes
        that copy moves; recorded in profiles/traffic.json under NAME with
        the hash of the kernel's sources (bench.py uses the record only
        while that hash matches).
"""
from __future__ import annotations

import argparse
import csv
import json
import os
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_BYTES = 512 << 20          # profile_run.py copy: a 512 MiB float32 tensor copied


def per_kernel(path):
    """{kernel name: {counter: [value per dispatch, ...]}}"""
    out = defaultdict(lambda: defaultdict(list))
    with open(path) as f:
        for r in csv.DictReader(f):
            out[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return out


def mean_of(path, kernel_sub, counter):
    vals = [v for k, cs in per_kernel(path).items() if kernel_sub in k for v in cs.get(counter, [])]
    if not vals:
        raise SystemExit("no %s for a kernel matching %r in %s" % (counter, kernel_sub, path))
    return sum(vals) / len(vals), len(vals)


def table(paths):
    lines = ["| kernel | dispatches | counter | mean per dispatch |", "|---|---|---|---|"]
    for p in paths:
        for k, cs in sorted(per_kernel(p).items()):
            for c, v in sorted(cs.items()):
                lines.append("| `%s` | %d | %s | %.1f |" % (k[:90], len(v), c, sum(v) / len(v)))
    return "\n".join(lines)


def trace(a):
    import statistics
    with open(a.csv) as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    dur = defaultdict(list)
    for r in rows:
        if a.kernel is None or a.kernel in r["Kernel_Name"]:
            dur[r["Kernel_Name"]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    lines = ["| kernel | calls | mean us | median us | min us | max us |", "|---|---|---|---|---|---|"]
    for k, v in sorted(dur.items(), key=lambda kv: -sum(kv[1])):
        if a.kernel is not None:
            v = v[a.skip:a.skip + a.first] if a.first else v[a.skip:]
        if not v:
            continue
        lines.append("| `%s` | %d | %.2f | %.2f | %.2f | %.2f |" % (
            k[:110], len(v), sum(v) / len(v), statistics.median(v), min(v), max(v)))
        if a.kernel is not None:
            lines.append("")
            lines.append("launch durations (us, dispatch order): " + ", ".join("%.1f" % x for x in v))
            lines.append("")
    return "\n".join(lines)


def traffic(a):
    sys.path.insert(0, ROOT)
    import bench
    cf, _ = mean_of(a.calib_fetch, "copyBuffer", "FETCH_SIZE")
    cw, _ = mean_of(a.calib_write, "copyBuffer", "WRITE_SIZE")
    ff, fw = COPY_BYTES / (cf * 1024.0), COPY_BYTES / (cw * 1024.0)
    f, n = mean_of(a.fetch, a.kernel, "FETCH_SIZE")
    w, _ = mean_of(a.write, a.kernel, "WRITE_SIZE")
    total = f * 1024.0 * ff + w * 1024.0 * fw
    path = os.path.join(ROOT, "profiles", "traffic.json")
    rec = json.load(open(path)) if os.path.exists(path) else {}
    rec["_calibration"] = {"copy_bytes": COPY_BYTES, "FETCH_SIZE_kib": cf, "WRITE_SIZE_kib": cw,
                           "fetch_factor": ff, "write_factor": fw}
    src_kernel = a.key.split("|")[0]
    rec[a.key] = {"bytes_per_launch": int(round(total)), "fetch_kib": f, "write_kib": w, "launches": n,
                  "algorithmic_bytes": a.algorithmic, "ratio_to_algorithmic": round(total / a.algorithmic, 3),
                  "source_hash": bench.kernel_source_hash(src_kernel), "command": a.command}
    with open(path, "w") as fh:
        json.dump(rec, fh, indent=1, sort_keys=True)
    print("%s: %.0f bytes per launch, %.3f x algorithmic" % (a.key, total, total / a.algorithmic))


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("table")
    t.add_argument("csv", nargs="+")
    tr = sub.add_parser("trace")
    tr.add_argument("csv")
    tr.add_argument("--kernel", default=None)
    tr.add_argument("--first", type=int, default=0)
    tr.add_argument("--skip", type=int, default=0)
    r = sub.add_parser("traffic")
    for n in ("fetch", "write", "calib_fetch", "calib_write", "kernel", "key", "command"):
        r.add_argument("--" + n.replace("_", "-"), required=True)
    r.add_argument("--algorithmic", type=int, required=True)
    a = ap.parse_args(argv)
    if a.cmd == "table":
        print(table(a.csv))
    elif a.cmd == "trace":
        print(trace(a))
    else:
        traffic(a)


if __name__ == "__main__":
    main()
