"""Refresh a committed profile summary (profiles/*.txt) and the traffic records
(profiles/traffic.json) from new rocprofv3 output of the commands the summary gives.

    python -m bit_quantized_routed_amd.prof_report decode ROW TAG PROFDIR SUMMARY
    python -m bit_quantized_routed_amd.prof_report prefill PROFDIR SUMMARY

PROFDIR holds what the summary's commands wrote (kt_TAG/kt_kernel_stats.csv,
pmc_TAG_FETCH_SIZE/c_counter_collection.csv, pmc_TAG_WRITE_SIZE/..., sq_*/p_...) and,
as TAG-named .json files, bench.py's JSON line of each run (kt_TAG.json: the
algorithmic bytes and touched experts, averaged over every rotated layer).  `decode`
rewrites the summary's numeric sections (the kernel trace table, the profiled step time, the FETCH_SIZE / WRITE_SIZE tables, the copy
calibration, the per-launch traffic) and keeps its prose; it also rewrites the two
traffic records of ROW (gate_up, down) with the kernel source's hash as the library
compiles it.  `prefill` rewrites the three kernel trace tables, the profiled step and
launch figures and the 15-bit instruction-counter lines of the prefill summary.
"""
import collections
import csv
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCE = "bit_quantized_routed_amd/csrc/ffn_mma.hip"
GENERATION = ("k_synth_normal", "k_quantize", "k_pack_expert")
HBM_PEAK = 8e12


def _stats_rows(path):
    rows = [r for r in csv.DictReader(open(path))]
    out = []
    for r in rows:
        name = r["Name"]
        bare = name[5:] if name.startswith("void ") else name
        if not bare.startswith("k_") or any(bare.startswith(g) for g in GENERATION):
            continue
        out.append(r)
    out.sort(key=lambda r: -float(r["TotalDurationNs"]))
    return out


def stats_table(path):
    lines = ["%-70s %7s %12s %12s %7s" % ("kernel", "calls", "total_us", "avg_us", "pct")]
    for r in _stats_rows(path):
        lines.append("%-70s %7s %12.1f %12.2f %7.2f" % (r["Name"][:70], r["Calls"], float(r["TotalDurationNs"]) / 1e3,
                                                        float(r["AverageNs"]) / 1e3, float(r["Percentage"])))
    return lines


def trace_avg_us(path, prefix):
    """Mean duration (us) over all dispatches of the kernels whose name starts with prefix."""
    tot = n = 0.0
    for r in _stats_rows(path):
        if r["Name"].startswith(prefix):
            tot += float(r["TotalDurationNs"])
            n += int(r["Calls"])
    return tot / n / 1e3 if n else None


def pmc_groups(path, counter):
    """{(name[:70], grid): [values]} of one counter."""
    g = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            g[(r["Kernel_Name"][:70], r["Grid_Size"])].append(float(r["Counter_Value"]))
    return g


def pmc_table(groups, counter):
    lines = ["%-70s %10s %s" % ("kernel", "grid", "counter: mean per dispatch (dispatches)")]
    for (name, grid), v in sorted(groups.items()):
        lines.append("%-70s %10s %s: %.1f (%d)" % (name, grid, counter, sum(v) / len(v), len(v)))
    return lines


def launch_mean(groups, prefix):
    """(names, grids, dispatches, mean value per dispatch) over the launches of one kind."""
    names, grids, vals = [], [], []
    for (name, grid), v in sorted(groups.items()):
        if name.startswith(prefix):
            names.append(name)
            grids.append(int(grid))
            vals += v
    return sorted(set(names)), sorted(set(grids)), len(vals), (sum(vals) / len(vals) if vals else None)


def calibration(fetch, write):
    """Counter factors from the 1 GiB device copy (the copy kernel with the largest write)."""
    cw = {k: v for k, v in write.items() if "copyBuffer" in k[0]}
    key = max(cw, key=lambda k: sum(cw[k]) / len(cw[k]))
    f = sum(fetch[key]) / len(fetch[key])
    w = sum(cw[key]) / len(cw[key])
    return {"bytes_read": 1 << 30, "bytes_written": 1 << 30, "fetch_kib": round(f, 1), "write_kib": round(w, 1),
            "fetch_factor": round(1048576.0 / f, 4), "write_factor": round(1048576.0 / w, 4)}


def source_hash():
    sys.path.insert(0, ROOT)
    import bench
    return hashlib.sha256(bench.library_source(open(os.path.join(ROOT, SOURCE)).read()).encode()).hexdigest()


def _replace_block(lines, start_pred, new, stop_pred=lambda l: not l.strip(), include_start=True):
    """Lines with the block that starts at the first line matching start_pred (through the
    line before the first later line matching stop_pred) replaced by new."""
    for i, l in enumerate(lines):
        if start_pred(l):
            j = i + 1
            while j < len(lines) and not stop_pred(lines[j]):
                j += 1
            return lines[:i] + new + lines[j:] if include_start else lines[:i + 1] + new + lines[j:]
    raise SystemExit("summary section not found")


def decode(row, tag, pdir, summary):
    kt = os.path.join(pdir, "kt_%s" % tag, "kt_kernel_stats.csv")
    fcsv = os.path.join(pdir, "pmc_%s_FETCH_SIZE" % tag, "c_counter_collection.csv")
    wcsv = os.path.join(pdir, "pmc_%s_WRITE_SIZE" % tag, "c_counter_collection.csv")
    ktj = json.loads(open(os.path.join(pdir, "kt_%s.json" % tag)).read().strip().splitlines()[-1])
    fetch, write = pmc_groups(fcsv, "FETCH_SIZE"), pmc_groups(wcsv, "WRITE_SIZE")
    cal = calibration(fetch, write)
    # the algorithmic bytes average every rotated layer: taken from the trace run (its
    # steps pass over all of them; a 5-step counter run leaves some layers unused)
    alg = ktj["roofline"]["algorithmic_bytes_by_launch"]
    touched = ktj["config"]["touched_experts_mean"]
    lines = open(summary).read().splitlines()
    lines = _replace_block(lines, lambda l: l.startswith("kernel ") and "calls" in l, stats_table(kt))
    lines = _replace_block(lines, lambda l: l.startswith("bench.py in this profiled run"),
                           ["bench.py in this profiled run: %.2f us per step (graph replay), eager %.2f us." % (
                               ktj["ms_per_step"] * 1e3, ktj["config"]["eager_ms_per_step"] * 1e3)])
    lines = _replace_block(lines, lambda l: l.startswith("FETCH_SIZE (KiB"), pmc_table(fetch, "FETCH_SIZE"),
                           stop_pred=lambda l: l.startswith("WRITE_SIZE (KiB"), include_start=False)
    lines = _replace_block(lines, lambda l: l.startswith("WRITE_SIZE (KiB"), pmc_table(write, "WRITE_SIZE"),
                           include_start=False)
    lines = _replace_block(lines, lambda l: l.startswith("Calibration:"), [
        "Calibration: the 1 GiB device copy reads and writes 1,048,576 KiB; the counters report",
        "FETCH %.1f KiB and WRITE %.1f KiB, so FETCH_SIZE is scaled by %.4f and WRITE_SIZE by %.4f" % (
            cal["fetch_kib"], cal["write_kib"], cal["fetch_factor"], cal["write_factor"]),
        "(profiles/traffic.json holds these per-launch figures for bench.py)."])
    per = ["Per launch (mean over the dispatches; touched experts per layer %.2f on average):" % touched]
    recs = {}
    sha = source_hash()
    for dom, prefix in (("gate_up", "void k_q2_mma<true"), ("down", "void k_q2_mma<false")):
        names, grids, nd, fk = launch_mean(fetch, prefix)
        _, _, _, wk = launch_mean(write, prefix)
        tb = (fk * cal["fetch_factor"] + wk * cal["write_factor"]) * 1024
        ab = alg[dom]
        us = trace_avg_us(kt, prefix)
        rate = ab / (us * 1e-6)
        per.append("  %-7s  traffic %.1f MB vs %.1f MB algorithmic (x%.3f); trace average %.2f us ->" % (
            dom, tb / 1e6, ab / 1e6, tb / ab, us))
        per.append("           %.2f TB/s algorithmic = %.3f of 8 TB/s" % (rate / 1e12, rate / HBM_PEAK))
        recs["%s/%s" % (row, dom)] = {
            "kernel": names[0] if len(names) == 1 else names, "workload": row, "grid": grids, "source": SOURCE,
            "source_sha256": sha, "dispatches": nd, "fetch_kib_per_dispatch": round(fk, 1),
            "write_kib_per_dispatch": round(wk, 1), "copy_calibration": cal, "bytes_per_launch": int(round(tb)),
            "algorithmic_bytes_per_launch": int(round(ab)), "touched_experts_mean": touched,
            "summary": os.path.relpath(summary, ROOT)}
    lines = _replace_block(lines, lambda l: l.startswith("Per launch (mean over"), per)
    open(summary, "w").write("\n".join(lines) + "\n")
    tpath = os.path.join(ROOT, "profiles", "traffic.json")
    allrec = json.load(open(tpath)) if os.path.exists(tpath) else {}
    allrec.update(recs)
    with open(tpath, "w") as f:
        json.dump(allrec, f, indent=1)
        f.write("\n")
    for k, r in recs.items():
        print(k, r["bytes_per_launch"], "x%.3f" % (r["bytes_per_launch"] / r["algorithmic_bytes_per_launch"]))


def _sq_lines(path):
    rows = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(path)):
        rows[(r["Kernel_Name"][:70], r["Grid_Size"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
    out = []
    for (name, grid), d in sorted(rows.items()):
        vals = ", ".join("%s: %.1f (%d)" % (c, sum(v) / len(v), len(v)) for c, v in sorted(d.items()))
        out.append("%-70s %10s %s" % (name, grid, vals))
    return out


def prefill(pdir, summary):
    lines = open(summary).read().splitlines()
    starts = [i for i, l in enumerate(lines) if l.startswith("kernel ") and "calls" in l]
    if len(starts) != 3:
        raise SystemExit("expected three trace tables")
    for i, tag in reversed(list(zip(starts, ("prefill", "prefillq8", "prefillq4")))):
        new = stats_table(os.path.join(pdir, "kt_%s" % tag, "kt_kernel_stats.csv"))
        j = i + 1
        while j < len(lines) and lines[j].startswith(("void ", "k_")):
            j += 1
        lines = lines[:i] + new + lines[j:]
    for tag, row, q8 in (("prefill", "prefill2048", False), ("prefillq8", "prefill2048:q8", True),
                         ("prefillq4", "prefill2048_q4", False)):
        js = json.loads(open(os.path.join(pdir, "kt_%s.json" % tag)).read().strip().splitlines()[-1])
        rf = js["roofline"]
        kt = os.path.join(pdir, "kt_%s" % tag, "kt_kernel_stats.csv")
        us = trace_avg_us(kt, "void k_q2_mma_pf<true")
        flops = rf["algorithmic_flops_per_launch"]
        peak = rf["peak"] * 1e12
        unit = "TOP/s (int8)" if q8 else "TFLOP/s"
        new = ["bench.py, %s, in its profiled run: %.3f ms per step (graph replay), eager %.3f ms; gate/up" % (
                   row, js["ms_per_step"], js["config"]["eager_ms_per_step"]),
               "  launch: %.1f GFLOP of useful work / %.3f ms (its own start/stop events, eager loop) = %.0f %s = %.3f of peak;" % (
                   flops / 1e9, rf["avg_launch_ms"], rf["achieved"], unit, rf["frac"]),
               "  trace average %.3f ms -> %.0f %s = %.3f of peak." % (
                   us / 1e3, flops / (us * 1e-6) / 1e12, unit, flops / (us * 1e-6) / peak)]
        lines = _replace_block(lines, lambda l, r=row: l.startswith("bench.py, %s, in its profiled run" % r), new,
                               stop_pred=lambda l: not l.startswith("  "))
    sq = _sq_lines(os.path.join(pdir, "sq_prefill_1", "p_counter_collection.csv")) + \
        _sq_lines(os.path.join(pdir, "sq_prefill_2", "p_counter_collection.csv"))
    lines = _replace_block(lines, lambda l: l.startswith("15-bit activations (ND = 2), 2-bit weights:"), sq,
                           stop_pred=lambda l: not l.startswith("void "), include_start=False)
    open(summary, "w").write("\n".join(lines) + "\n")


if __name__ == "__main__":
    if sys.argv[1] == "decode":
        decode(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5])
    elif sys.argv[1] == "prefill":
        prefill(sys.argv[2], sys.argv[3])
    else:
        raise SystemExit(__doc__)
