"""Summarise rocprofv3 CSV output into the short text/JSON files kept under
profiles/.

  kernel-stats:  python -m bf16_gemm_decode_amd.profile_summary stats \
                     <run_kernel_stats.csv> <out.txt> --command "<rocprofv3 command>" \
                     [--trace <run_kernel_trace.csv> --timed <kernel substring>:<skip>:<count> ...]
  mfma:          python -m bf16_gemm_decode_amd.profile_summary mfma \
                     --util-csv <csv> --counts-csv <csv> --kernel label=<substring>:<FLOP> ... \
                     --source <files...> --out <out.json> --commands "<cmd>" ...
  sweep-mfma:    python -m bf16_gemm_decode_amd.profile_summary sweep-mfma \
                     --util-csv <csv> --sweep-json <sweep stdout> --out <out.md> --command "<cmd>"
  counters:      python -m bf16_gemm_decode_amd.profile_summary counters \
                     --csv <counter_collection.csv> ... --kernel label=<substring> ... \
                     --source <files...> --out <out.json> --commands "<cmd>" ...
  traffic:       python -m bf16_gemm_decode_amd.profile_summary traffic \
                     --fetch <csv> --fetch-cal <csv> --write <csv> --write-cal <csv> \
                     --kernel <name substring> --source <source files...> \
                     --out <out.json> --commands "<cmd>" ...

The traffic mode averages FETCH_SIZE and WRITE_SIZE (KiB per dispatch) over
the matching kernel's dispatches and scales each by what the same counter
reads for the plain 1 GiB device copy of `bench.py --copy-calibration`
(profiled with the same counter), so that beyond_l2_bytes_per_launch (the
requests that leave L2 for the MALL or HBM) is in true bytes.  It records a SHA-256 over the sources that decide what the kernel
does (source_digest), so that a later change of them invalidates the figure.
"""
import argparse
import collections
import csv
import hashlib
import json
import os
import sys

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
# the sources whose change invalidates a kernel's recorded counters
GEMM_SOURCES = ["gemm.hip", "api.hip", "kernels.hpp", "tile_map.hpp", "common.hpp", "dma.hpp"]
GEMV_SOURCES = ["gemv.hip", "skinny.hip", "batch.hip", "wide.hip", "api.hip", "kernels.hpp", "common.hpp", "dma.hpp"]
ATTENTION_SOURCES = ["attention.hip", "api.hip", "kernels.hpp", "common.hpp"]


def source_digest(names):
    """SHA-256 over the named csrc/ files (name and content, in order)."""
    h = hashlib.sha256()
    for n in names:
        h.update(n.encode() + b"\0")
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def stats(args):
    rows = _rows(args.csv)
    keys = list(rows[0].keys()) if rows else []
    with open(args.out, "w") as o:
        o.write("# rocprofv3 kernel statistics\n# command: %s\n" % args.command)
        o.write("# columns: %s\n" % ", ".join(keys))
        for r in rows:
            name = r.get("Name", "")
            if args.filter and not any(f in name for f in args.filter):
                continue
            o.write(", ".join(str(r[k]) for k in keys) + "\n")
        # the timed region of bench.py: the kernel's dispatches after the
        # warm-up ones, in dispatch order, from the kernel trace
        for spec in args.timed or []:
            substr, skip, count = spec.rsplit(":", 2)
            d = sorted((int(r["Dispatch_Id"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
                       for r in _rows(args.trace) if substr in r["Kernel_Name"])
            sel = [t for _, t in d[int(skip):int(skip) + int(count)]]
            if not sel:
                sys.exit("no dispatches of %r in %s" % (substr, args.trace))
            o.write("# timed region: %s dispatches %d..%d of %d: average %.1f ns, min %d, max %d\n"
                    % (substr, int(skip), int(skip) + len(sel) - 1, len(d), sum(sel) / len(sel),
                       min(sel), max(sel)))
        # what bench.py itself reported in the profiled run
        if args.bench_json:
            with open(args.bench_json) as f:
                for line in f:
                    if line.startswith("{") and '"roofline"' in line:
                        b = json.loads(line)
                        o.write("# bench.py in the same run: GEMM avg_launch_ms %s (HIP events, timed region), "
                                "GEMV avg_launch_us %s\n" % (b["roofline"]["avg_launch_ms"],
                                                            b["gemv"]["avg_launch_us"]))
    print(open(args.out).read())


def _counter_per_dispatch(path, counter, substr):
    per = collections.defaultdict(float)
    names = {}
    for r in _rows(path):
        if r["Counter_Name"] != counter:
            continue
        per[r["Dispatch_Id"]] += float(r["Counter_Value"])
        names[r["Dispatch_Id"]] = r["Kernel_Name"]
    hit = [v for d, v in per.items() if substr in names[d]]
    return hit, per, names


def _median(v):
    v = sorted(v)
    return v[len(v) // 2]


def traffic(args):
    out = {"commands": args.commands, "kernel": args.kernel}
    for counter, path, cal in (("FETCH_SIZE", args.fetch, args.fetch_cal),
                               ("WRITE_SIZE", args.write, args.write_cal)):
        vals, _, _ = _counter_per_dispatch(path, counter, args.kernel)
        _, per, names = _counter_per_dispatch(cal, counter, "")
        copy = [v for d, v in per.items() if "copy" in names[d].lower()]
        if not vals or not copy:
            sys.exit("no %s values for kernel %r in %s or for a copy kernel in %s"
                     % (counter, args.kernel, path, cal))
        # the copy moves 1 GiB each way: its reading in KiB against the true
        # 1 GiB gives this counter's factor to bytes
        copy_kib = _median(copy)
        scale = (1 << 30) / (copy_kib * 1024.0)
        kib = sum(vals) / len(vals)
        out[counter.lower()] = {"kib_per_dispatch_raw": kib, "dispatches": len(vals),
                                "copy_kib_raw": copy_kib, "scale_to_bytes": scale,
                                "bytes_per_launch": kib * 1024.0 * scale}
    # FETCH_SIZE and WRITE_SIZE count the requests that leave L2 (served by
    # the MALL or by HBM), not HBM transfers alone
    out["beyond_l2_bytes_per_launch"] = (out["fetch_size"]["bytes_per_launch"] +
                                         out["write_size"]["bytes_per_launch"])
    out["kernel_sources"] = args.source
    out["kernel_sources_sha256"] = source_digest(args.source)
    with open(args.out, "w") as o:
        json.dump(out, o, indent=1)
    print(json.dumps(out, indent=1))


def counters(args):
    """Every counter of the given --pmc runs, per kernel label: mean, min and
    max over the matching dispatches, with their average duration."""
    out = {"commands": args.commands, "kernels": {}}
    rows = [r for path in args.csv for r in _rows(path)]
    for spec in args.kernel:
        label, substr = spec.split("=", 1)
        per = collections.defaultdict(dict)     # counter -> {(file row set, dispatch): value}
        dur = {}
        for r in rows:
            if substr not in r["Kernel_Name"]:
                continue
            key = (r["Counter_Name"], r["Dispatch_Id"], r["Kernel_Name"])
            per[r["Counter_Name"]][key] = float(r["Counter_Value"])
            dur[(r["Dispatch_Id"], r["Kernel_Name"], r["Counter_Name"])] = \
                int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        if not per:
            sys.exit("no counter rows for kernel %r" % substr)
        k = {"kernel_name_contains": substr, "counters": {}}
        for name, vals in sorted(per.items()):
            v = list(vals.values())
            k["counters"][name] = {"mean": sum(v) / len(v), "min": min(v), "max": max(v),
                                   "dispatches": len(v)}
        d = list(dur.values())
        k["avg_duration_ns"] = sum(d) / len(d)
        out["kernels"][label] = k
    out["kernel_sources"] = args.source
    out["kernel_sources_sha256"] = source_digest(args.source)
    with open(args.out, "w") as o:
        json.dump(out, o, indent=1)
    print(json.dumps(out, indent=1))


def _per_dispatch(path, counter, substr):
    """{dispatch id: (value, duration in ns)} of one counter for the
    dispatches whose kernel name contains substr (rocprofv3's CSV holds one
    row per dispatch and counter, instances already combined)."""
    out = {}
    for r in _rows(path):
        if r["Counter_Name"] == counter and substr in r["Kernel_Name"]:
            out[r["Dispatch_Id"]] = (float(r["Counter_Value"]),
                                     int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return out


def mfma(args):
    """MFMA utilisation per kernel from a --pmc MfmaUtil run (rocprofv3's
    derived counter: MFMA-busy SIMD cycles / (GPU-active cycles x SIMDs), in
    %), and from a --pmc run of the raw counters the MFMA FLOP per dispatch
    (SQ_INSTS_VALU_MFMA_MOPS_F16 + _BF16, units of 512 FLOP) against the
    algorithmic count, and GRBM_GUI_ACTIVE per XCD over the dispatch time
    (the clock the kernel ran at)."""
    out = {"commands": args.commands, "kernels": {}}
    for spec in args.kernel:
        label, rest = spec.split("=", 1)
        substr, flop = rest.rsplit(":", 1)
        util = _per_dispatch(args.util_csv, "MfmaUtil", substr)
        if not util:
            sys.exit("no MfmaUtil values for %r in %s" % (substr, args.util_csv))
        u = [v for v, _ in util.values()]
        row = {"kernel_name_contains": substr, "dispatches": len(u),
               "mfma_util_percent": {"mean": sum(u) / len(u), "min": min(u), "max": max(u)}}
        mops = [_per_dispatch(args.counts_csv, c, substr) for c in
                ("SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_VALU_MFMA_MOPS_BF16")]
        act = _per_dispatch(args.counts_csv, "GRBM_GUI_ACTIVE", substr)
        if act:
            ghz = [v / args.xcds / t for v, t in act.values()]
            row["gui_active_ghz_per_xcd"] = sum(ghz) / len(ghz)
            if float(flop) > 0:   # 16-bit kernels: the MOPS counters cover them
                f = [sum(m.get(d, (0.0, 0))[0] for m in mops) * 512.0 for d in act]
                row["mfma_flop_per_dispatch"] = sum(f) / len(f)
                row["algorithmic_flop_per_dispatch"] = float(flop)
                row["mfma_flop_over_algorithmic"] = (sum(f) / len(f)) / float(flop)
        out["kernels"][label] = row
    out["kernel_sources"] = args.source
    out["kernel_sources_sha256"] = source_digest(args.source)
    with open(args.out, "w") as o:
        json.dump(out, o, indent=1)
    print(json.dumps(out, indent=1))


def sweep_mfma(args):
    """MfmaUtil of every configuration of a sweep.py run profiled with
    --pmc MfmaUtil.  sweep.py launches each configuration's GEMM 1 + warmup
    + reps times, in the order of its JSON lines; the GEMM dispatches (kernel
    names containing 'gemm_', in dispatch order) are cut into groups of that
    size and the timed ones (the last reps of each group) averaged."""
    util = {}
    names = {}
    for r in _rows(args.util_csv):
        if r["Counter_Name"] == "MfmaUtil" and "gemm_" in r["Kernel_Name"]:
            util[int(r["Dispatch_Id"])] = float(r["Counter_Value"])
            names[int(r["Dispatch_Id"])] = r["Kernel_Name"]
    order = sorted(util)
    cfgs = [json.loads(l) for l in open(args.sweep_json) if l.startswith("{")]
    per = 1 + args.warmup + args.reps
    if len(order) != per * len(cfgs):
        sys.exit("%d GEMM dispatches for %d configurations of %d" % (len(order), len(cfgs), per))
    with open(args.out, "w") as o:
        o.write("# MfmaUtil per configuration (rocprofv3 derived counter: MFMA-busy SIMD cycles over\n"
                "# GPU-active cycles x SIMDs), mean over each configuration's %d timed dispatches\n" % args.reps)
        o.write("# command: %s\n" % args.command)
        o.write("# sweep.py times (same run, under the counters): ms and TFLOP/s as it printed them\n\n")
        o.write("| shape | dtype | A layout | tile | tile_mnk | GROUP_M | ms | TFLOP/s | MfmaUtil % |\n")
        o.write("|---|---|---|---|---|---|---|---|---|\n")
        for i, c in enumerate(cfgs):
            ids = order[i * per:(i + 1) * per][1 + args.warmup:]
            u = [util[d] for d in ids]
            o.write("| %s | %s | %s | %d | %s | %d | %s | %s | %.1f |\n" % (
                "x".join(map(str, c["shape"])), c["dtype"], c["a_layout"], c["tile"],
                "x".join(map(str, c["tile_mnk"])), c["group_m"], c["ms"], c["tflops"], sum(u) / len(u)))
    print(open(args.out).read())


def main(argv=None):
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="mode", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("out")
    s.add_argument("--command", required=True)
    s.add_argument("--filter", nargs="*")
    s.add_argument("--trace", help="the run's kernel-trace CSV, for --timed")
    s.add_argument("--bench-json", help="stdout of the profiled bench.py run")
    s.add_argument("--timed", nargs="*",
                   help="<kernel name substring>:<dispatches to skip>:<count>: average over those dispatches")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--fetch-cal", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--write-cal", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--source", nargs="+", required=True,
                   help="csrc/ file names, e.g. the GEMM_SOURCES list")
    t.add_argument("--out", required=True)
    t.add_argument("--commands", nargs="+", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("--util-csv", required=True, help="counter CSV of a --pmc MfmaUtil run")
    m.add_argument("--counts-csv", required=True,
                   help="counter CSV of a --pmc GRBM_GUI_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_F16 _BF16 run")
    m.add_argument("--kernel", nargs="+", required=True,
                   help="label=<kernel name substring>:<algorithmic FLOP per dispatch, 0 for 8-bit>")
    m.add_argument("--xcds", type=int, default=8)
    m.add_argument("--source", nargs="+", required=True)
    m.add_argument("--out", required=True)
    m.add_argument("--commands", nargs="+", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--csv", nargs="+", required=True, help="counter_collection CSVs of --pmc runs")
    c.add_argument("--kernel", nargs="+", required=True, help="label=<kernel name substring>")
    c.add_argument("--source", nargs="+", required=True)
    c.add_argument("--out", required=True)
    c.add_argument("--commands", nargs="+", required=True)
    w = sub.add_parser("sweep-mfma")
    w.add_argument("--util-csv", required=True)
    w.add_argument("--sweep-json", required=True, help="stdout of the profiled sweep.py run")
    w.add_argument("--warmup", type=int, default=3)
    w.add_argument("--reps", type=int, default=10)
    w.add_argument("--out", required=True)
    w.add_argument("--command", required=True)
    a = p.parse_args(argv)
    {"stats": stats, "traffic": traffic, "mfma": mfma, "sweep-mfma": sweep_mfma,
     "counters": counters}[a.mode](a)


if __name__ == "__main__":
    main()
