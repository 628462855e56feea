"""Summaries of rocprofv3 output for the files under profiles/.

    python -m w4a16_decode_amd.profiling stats  <kernel_stats.csv> [name-filter]
    python -m w4a16_decode_amd.profiling counters <counter_collection.csv> <name-filter>
    python -m w4a16_decode_amd.profiling traffic --fetch F.csv --write W.csv --cal-fetch CF.csv
                                                   --cal-write CW.csv --cal-bytes N --kernel FILTER
    python -m w4a16_decode_amd.profiling split <kernel_trace.csv> <name-filter> <threshold_us> [label_below label_above]

`split` divides the launches of the kernels matching the filter at a duration
threshold (two matrices that share one kernel instance, e.g. the fused gate/up and
q/k/v GEMVs) and prints each side's count and average duration; the line
`<label_above>_avg_us_rocprof: X` is what bench.py reads back.

`traffic` turns FETCH_SIZE / WRITE_SIZE (KiB per dispatch) into bytes per launch,
each scaled by what the same counter reports for a plain device copy of a known
size (the copy reads and writes cal-bytes each).

The kernel fingerprint (kernel_fingerprint) hashes the GEMV sources with comments and
whitespace removed (the code the compiler sees); a figure recorded under profiles/ is
only used while it matches.
"""

from __future__ import annotations

import csv
import hashlib
import os
import statistics
import sys
from collections import defaultdict

from .build import code_only

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ("csrc/q4_gemm.hip", "csrc/q4_device.h")


def kernel_fingerprint(sources=None) -> str:
    """Hash of the GEMV kernel sources' code (comments and layout ignored)."""
    h = hashlib.sha256()
    for path in sources or [os.path.join(HERE, rel) for rel in KERNEL_SOURCES]:
        with open(path, encoding="utf-8") as f:
            h.update(code_only(f.read()).encode())
    return h.hexdigest()[:16]


def _short(name: str, n: int = 110) -> str:
    return name if len(name) <= n else name[: n - 3] + "..."


def kernel_stats(path: str, filt: str = "") -> list[dict]:
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if filt in r["Name"]:
                rows.append({"name": r["Name"], "calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3,
                             "min_us": float(r["MinNs"]) / 1e3, "max_us": float(r["MaxNs"]) / 1e3,
                             "pct": float(r["Percentage"])})
    rows.sort(key=lambda r: -r["pct"])
    return rows


def counters(path: str, filt: str) -> dict:
    vals = defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            if filt in r["Kernel_Name"]:
                vals[r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: statistics.mean(v) for k, v in vals.items()}


def traffic(fetch_csv, write_csv, cal_fetch_csv, cal_write_csv, cal_bytes: int, kernel: str,
            cal_kernel: str = "copyBuffer") -> dict:
    f_k = counters(fetch_csv, kernel)["FETCH_SIZE"]
    w_k = counters(write_csv, kernel)["WRITE_SIZE"]
    f_c = counters(cal_fetch_csv, cal_kernel)["FETCH_SIZE"]
    w_c = counters(cal_write_csv, cal_kernel)["WRITE_SIZE"]
    f_scale = cal_bytes / (f_c * 1024)
    w_scale = cal_bytes / (w_c * 1024)
    return {"fetch_bytes": f_k * 1024 * f_scale, "write_bytes": w_k * 1024 * w_scale,
            "fetch_scale": f_scale, "write_scale": w_scale,
            "bytes": f_k * 1024 * f_scale + w_k * 1024 * w_scale}


def split_durations(path: str, filt: str, threshold_us: float) -> tuple[list[float], list[float]]:
    below, above = [], []
    with open(path) as f:
        for r in csv.DictReader(f):
            if filt in r["Kernel_Name"]:
                d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                (above if d >= threshold_us else below).append(d)
    return below, above


def main(argv):
    if not argv:
        print(__doc__)
        return 2
    cmd = argv[0]
    if cmd == "stats":
        for r in kernel_stats(argv[1], argv[2] if len(argv) > 2 else ""):
            print(f"{r['calls']:6d} calls  avg {r['avg_us']:9.2f} us  min {r['min_us']:9.2f}  max {r['max_us']:9.2f}"
                  f"  {r['pct']:5.1f}%  {_short(r['name'])}")
    elif cmd == "counters":
        for k, v in sorted(counters(argv[1], argv[2]).items()):
            print(f"{k:32s} {v:16.1f}")
    elif cmd == "traffic":
        opts = dict(zip(argv[1::2], argv[2::2]))
        t = traffic(opts["--fetch"], opts["--write"], opts["--cal-fetch"], opts["--cal-write"],
                    int(opts["--cal-bytes"]), opts["--kernel"])
        for k, v in t.items():
            print(f"{k}: {v:.6g}")
        print(f"kernel_fingerprint: {kernel_fingerprint()}")
    elif cmd == "split":
        below, above = split_durations(argv[1], argv[2], float(argv[3]))
        lb, la = (argv[4], argv[5]) if len(argv) > 5 else ("below", "above")
        for label, v in ((lb, below), (la, above)):
            if v:
                print(f"{label}: {len(v)} launches, avg {statistics.mean(v):.2f} us, median {statistics.median(v):.2f} us")
                print(f"{label}_avg_us_rocprof: {statistics.mean(v):.3f}")
        print(f"kernel_fingerprint: {kernel_fingerprint()}")
    elif cmd == "fingerprint":
        print(kernel_fingerprint())
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
