"""Summaries of rocprofv3 output (CSV format) for the kernels of this library.

  python -m mhc_hyper_connection_02_amd.profiling stats <trace_dir> --cmd "<command>"
      [--json-kernel <substr> --json-out <json> --source-hash H]
      per-kernel dispatch count and duration from a ``--kernel-trace --stats`` run (and
      one kernel's figures as JSON, which bench.py reports beside its own timing)
  python -m mhc_hyper_connection_02_amd.profiling mfma <dir> [<dir> ...] --match <substr>
      --cmd "<commands>"
      per (kernel, grid size): mean of every counter found in the ``--pmc`` runs' CSVs
      (e.g. SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE,
      MfmaUtil) and the mean dispatch duration of those runs
  python -m mhc_hyper_connection_02_amd.profiling traffic --fetch <dir> --write <dir>
      --cal-fetch <dir> --cal-write <dir> --cal-bytes N --kernel <substring>
      --block B --source-hash H --cmd "<commands>" --out <json>
      HBM bytes per launch of one kernel from two ``--pmc`` runs (FETCH_SIZE, then
      WRITE_SIZE, KiB per dispatch), each scaled by what the same counter reads for a
      plain device copy of cal-bytes bytes.

Nothing here touches the GPU; it only reads the CSV files rocprofv3 wrote.
"""

import argparse
import collections
import csv
import glob
import json
import os
import sys


def _find(d, suffix):
    hits = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[0]


def kernel_stats(trace_dir):
    """[(name, calls, avg_ns, median_ns, min_ns, max_ns)] from the kernel trace, longest
    total first."""
    rows = list(csv.DictReader(open(_find(trace_dir, "kernel_trace.csv"))))
    agg = collections.defaultdict(list)
    for r in rows:
        agg[r["Kernel_Name"]].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out = []
    for k, v in agg.items():
        v = sorted(v)
        med = v[len(v) // 2] if len(v) % 2 else (v[len(v) // 2 - 1] + v[len(v) // 2]) / 2
        out.append((k, len(v), sum(v) / len(v), med, v[0], v[-1]))
    return sorted(out, key=lambda t: -t[1] * t[2])


def counter_mean(pmc_dir, counter, kernel_substring):
    """Mean per-dispatch value of a counter over the dispatches of kernels matching."""
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(_find(pmc_dir, "counter_collection.csv")))
            if r["Counter_Name"] == counter and kernel_substring in r["Kernel_Name"]]
    if not vals:
        raise ValueError(f"no {counter} samples for kernels matching {kernel_substring!r}")
    return sum(vals) / len(vals), len(vals)


def counters_by_dispatch_shape(dirs, matches):
    """{(kernel, grid_size): {counter: [values], "_dur_ns": [durations]}} over the counter
    CSVs of the given ``--pmc`` runs, for kernels whose name contains one of `matches`."""
    out = collections.defaultdict(lambda: collections.defaultdict(list))
    for d in dirs:
        for r in csv.DictReader(open(_find(d, "counter_collection.csv"))):
            name = r["Kernel_Name"]
            if not any(m in name for m in matches):
                continue
            key = (name, int(r["Grid_Size"]))
            out[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
            out[key]["_dur_ns"].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("trace_dir")
    s.add_argument("--cmd", required=True)
    s.add_argument("--json-kernel", help="with --json-out: the kernel (name substring) whose "
                   "durations go to the JSON summary")
    s.add_argument("--json-out")
    s.add_argument("--source-hash", help="hash of the kernel sources the trace was taken on")
    m = sub.add_parser("mfma")
    m.add_argument("dirs", nargs="+")
    m.add_argument("--match", action="append", required=True)
    m.add_argument("--cmd", required=True)
    t = sub.add_parser("traffic")
    for k in ("fetch", "write", "cal_fetch", "cal_write", "kernel", "source_hash", "cmd", "out"):
        t.add_argument("--" + k.replace("_", "-"), required=True)
    t.add_argument("--cal-bytes", type=int, required=True)
    t.add_argument("--block", type=int, required=True)
    a = ap.parse_args(argv)

    if a.what == "mfma":
        print(f"# rocprofv3 --pmc counters per (kernel, grid size), mean per dispatch\n"
              f"# commands: {a.cmd}\n")
        for (name, grid), cs in sorted(counters_by_dispatch_shape(a.dirs, a.match).items()):
            durs = cs.pop("_dur_ns")
            print(f"{name}\n  grid {grid} threads, {len(durs)} counter samples, "
                  f"mean duration under --pmc {sum(durs) / len(durs) / 1e3:.2f} us")
            for c, v in sorted(cs.items()):
                print(f"  {c:32s} {sum(v) / len(v):14.6g}  ({len(v)} dispatches)")
        return 0

    if a.what == "stats":
        print(f"# rocprofv3 kernel trace: per-dispatch duration\n# command: {a.cmd}\n")
        print(f"{'calls':>6} {'avg_us':>9} {'median_us':>9} {'min_us':>9} {'max_us':>9}  kernel")
        stats = kernel_stats(a.trace_dir)
        for name, n, avg, med, mn, mx in stats:
            print(f"{n:6d} {avg / 1e3:9.3f} {med / 1e3:9.3f} {mn / 1e3:9.3f} {mx / 1e3:9.3f}  {name}")
        if a.json_out:
            hit = [t for t in stats if a.json_kernel in t[0]]
            if len(hit) != 1:
                raise ValueError(f"{len(hit)} kernels match {a.json_kernel!r}")
            name, n, avg, med, mn, mx = hit[0]
            with open(a.json_out, "w") as f:
                json.dump({"kernel": name, "dispatches": n, "avg_us": round(avg / 1e3, 3),
                           "median_us": round(med / 1e3, 3), "min_us": round(mn / 1e3, 3),
                           "max_us": round(mx / 1e3, 3), "source_hash": a.source_hash,
                           "command": a.cmd}, f, indent=1)
                f.write("\n")
        return 0

    fk, nf = counter_mean(a.fetch, "FETCH_SIZE", a.kernel)
    wk, nw = counter_mean(a.write, "WRITE_SIZE", a.kernel)
    cf, _ = counter_mean(a.cal_fetch, "FETCH_SIZE", "copyBuffer")
    cw, _ = counter_mean(a.cal_write, "WRITE_SIZE", "copyBuffer")
    sf = a.cal_bytes / (cf * 1024.0)
    sw = a.cal_bytes / (cw * 1024.0)
    res = {
        "kernel": a.kernel, "block": a.block, "source_hash": a.source_hash,
        "fetch_kib_per_dispatch": round(fk, 1), "write_kib_per_dispatch": round(wk, 1),
        "dispatches": [nf, nw],
        "copy_calibration": {"bytes": a.cal_bytes, "fetch_kib": round(cf, 1),
                             "write_kib": round(cw, 1), "fetch_scale": round(sf, 4),
                             "write_scale": round(sw, 4)},
        "hbm_read_bytes_per_launch": int(fk * 1024 * sf),
        "hbm_write_bytes_per_launch": int(wk * 1024 * sw),
        "hbm_bytes_per_launch": int(fk * 1024 * sf + wk * 1024 * sw),
        "commands": a.cmd,
    }
    with open(a.out, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    json.dump(res, sys.stdout, indent=1)
    print()
    return 0


if __name__ == "__main__":
    sys.exit(main())
