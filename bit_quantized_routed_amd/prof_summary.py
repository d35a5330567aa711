"""Summaries of rocprofv3 CSV output (kernel trace statistics and PMC counters).

    python -m bit_quantized_routed_amd.prof_summary stats <kernel_stats.csv>
    python -m bit_quantized_routed_amd.prof_summary pmc <counter_collection.csv> [regex]
    python -m bit_quantized_routed_amd.prof_summary timeline <kernel_trace.csv> [n]

`pmc` prints, per kernel name (and grid size), the mean of each counter per
dispatch, e.g. FETCH_SIZE / WRITE_SIZE in KiB."""
import collections
import csv
import re
import sys


def stats(path):
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    print("%-70s %7s %12s %12s %7s" % ("kernel", "calls", "total_us", "avg_us", "pct"))
    for r in rows:
        name = r["Name"][:70]
        print("%-70s %7s %12.1f %12.2f %7.2f" % (name, r["Calls"], float(r["TotalDurationNs"]) / 1e3,
                                                 float(r["AverageNs"]) / 1e3, float(r["Percentage"])))


def pmc(path, pattern=None):
    rows = list(csv.DictReader(open(path)))
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in rows:
        name = r["Kernel_Name"]
        if pattern and not re.search(pattern, name):
            continue
        agg[(name[:70], r["Grid_Size"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    print("%-70s %10s %s" % ("kernel", "grid", "counter: mean per dispatch (dispatches)"))
    for (name, grid), d in sorted(agg.items()):
        vals = ", ".join("%s: %.1f (%d)" % (c, sum(v) / len(v), len(v)) for c, v in sorted(d.items()))
        print("%-70s %10s %s" % (name, grid, vals))


def timeline(path, n=40):
    """The last n dispatches in start order: duration and idle gap before each."""
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    rows = rows[-n:]
    print("%-60s %10s %10s" % ("kernel", "dur_us", "gap_us"))
    prev = None
    for r in rows:
        t0, t1 = int(r["Start_Timestamp"]), int(r["End_Timestamp"])
        gap = (t0 - prev) / 1e3 if prev is not None else 0.0
        print("%-60s %10.2f %10.2f" % (r["Kernel_Name"][:60], (t1 - t0) / 1e3, gap))
        prev = t1


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        stats(sys.argv[2])
    elif sys.argv[1] == "timeline":
        timeline(sys.argv[2], int(sys.argv[3]) if len(sys.argv) > 3 else 40)
    else:
        pmc(sys.argv[2], sys.argv[3] if len(sys.argv) > 3 else None)
