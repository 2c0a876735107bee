"""Summaries of rocprofv3 output for the profiles folder.

  python -m top_sparse_attention_ls_amd.profsum stats KERNEL_STATS_CSV \\
      --out profiles/NAME.md --cmd "the rocprofv3 command"
      per-kernel calls / average / total duration of the library's kernels

  python -m top_sparse_attention_ls_amd.profsum traffic \\
      --fetch FETCH_COUNTER_CSV --write WRITE_COUNTER_CSV --copy-mib N \\
      --workload NAME --cmd-fetch "..." --cmd-write "..."
      HBM bytes per launch of the coarse scoring kernel from FETCH_SIZE and
      WRITE_SIZE (KiB per dispatch), each scaled by what the same counter
      reads for the plain N MiB device copy that bench.py --copy-calib runs
      last.  Writes profiles/k_coarse.NAME.traffic.json (read by bench.py,
      keyed to the kernel's source hash) and a .md beside it.

  python -m top_sparse_attention_ls_amd.profsum counters PASS_CSV ... \
      --copy-mib N --workload NAME --out profiles/NAME.md --cmd "..." ...
      every counter of every pass (one rocprofv3 --pmc run each), averaged
      per launch for each of the library's kernels; FETCH_SIZE / WRITE_SIZE
      scaled by the calibration copy as above and set against each kernel's
      algorithmic bytes per launch at that workload.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
# the coarse kernel and every header it includes
COARSE_SOURCES = ["k_index.hip", "ls_bucket.h", "ls_device.h", "ls_launch.h"]
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def coarse_kernel_sha() -> str:
    h = hashlib.sha256()
    for f in COARSE_SOURCES:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    n = name[5:] if name.startswith("void ") else name
    return n.split("(")[0]


def cmd_stats(args):
    rows = list(csv.DictReader(open(args.csv)))
    ours = [r for r in rows if short_name(r["Name"]).startswith("ls::")]
    ours.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = ["# %s" % args.title, "", "Command:", "", "```", args.cmd, "```", "",
             "| kernel | calls | avg us | min us | max us | total us |",
             "|---|---:|---:|---:|---:|---:|"]
    for r in ours:
        lines.append("| `%s` | %s | %.2f | %.2f | %.2f | %.1f |" % (
            short_name(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3,
            float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
            float(r["TotalDurationNs"]) / 1e3))
    if args.note:
        lines += ["", args.note]
    open(args.out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _counter_rows(path, counter):
    out = []
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            out.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    out.sort()
    return out


def _scaled(path, counter, copy_kib, kernel):
    rows = _counter_rows(path, counter)
    copies = [v for _, n, v in rows if n == COPY_KERNEL][-2:]
    if len(copies) < 2:
        raise SystemExit("no calibration copy found in %s" % path)
    cal = sum(copies) / len(copies)
    if not (0.5 * copy_kib < cal < 2.0 * copy_kib):
        raise SystemExit("%s of the copy reads %.0f KiB, expected about %.0f" %
                         (counter, cal, copy_kib))
    factor = copy_kib / cal
    vals = [v for _, n, v in rows if short_name(n).startswith("ls::" + kernel)]
    if not vals:
        raise SystemExit("no %s dispatch in %s" % (kernel, path))
    # the first launches of a run can see cold TLBs; use the later ones
    steady = vals[len(vals) // 2:] if len(vals) > 2 else vals
    avg_kib = sum(steady) / len(steady)
    return {"counter": counter, "raw_kib_per_launch": avg_kib, "launches": len(vals),
            "copy_raw_kib": cal, "copy_expected_kib": copy_kib, "factor": factor,
            "bytes_per_launch": avg_kib * factor * 1024.0}


def cmd_traffic(args):
    copy_kib = args.copy_mib * 1024.0
    f = _scaled(args.fetch, "FETCH_SIZE", copy_kib, "k_coarse")
    w = _scaled(args.write, "WRITE_SIZE", copy_kib, "k_coarse")
    total = f["bytes_per_launch"] + w["bytes_per_launch"]
    res = {"kernel": "k_coarse", "workload": args.workload, "kernel_sha": coarse_kernel_sha(),
           "bytes_per_launch": round(total), "fetch": f, "write": w,
           "algorithmic_bytes_per_launch": args.algorithmic,
           "commands": [args.cmd_fetch, args.cmd_write]}
    base = os.path.join(ROOT, "profiles", "k_coarse.%s.traffic" % args.workload)
    json.dump(res, open(base + ".json", "w"), indent=1)
    lines = ["# k_coarse HBM traffic, %s" % args.workload, "",
             "Commands (one counter per pass):", "", "```", args.cmd_fetch, args.cmd_write,
             "```", "",
             "| counter | raw KiB / launch | copy raw KiB | copy expected KiB | factor | "
             "scaled bytes / launch |", "|---|---:|---:|---:|---:|---:|"]
    for c in (f, w):
        lines.append("| %s | %.0f | %.0f | %.0f | %.4f | %.0f |" % (
            c["counter"], c["raw_kib_per_launch"], c["copy_raw_kib"], c["copy_expected_kib"],
            c["factor"], c["bytes_per_launch"]))
    lines += ["", "Total HBM bytes per launch: %.0f" % total]
    if args.algorithmic:
        lines.append("Algorithmic bytes per launch: %d (ratio %.3f)" %
                     (args.algorithmic, total / args.algorithmic))
    lines.append("Kernel source hash: %s" % res["kernel_sha"])
    open(base + ".md", "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


# Algorithmic bytes per launch of each decode-step kernel, from the parts of
# the step's byte count (bench.algorithmic_bytes): the workload's own reads
# and writes, never the workspace.
KERNEL_PARTS = {
    "k_coarse": ("coarse_keys", "idx_q_w"),
    "k_refine": ("refine_keys", "slot_table"),
    "k_hot_gather": ("miss_read", "miss_write"),
    "k_attn_mfma": ("kv_rows", "attn_q"),
    "k_attn_fused": ("kv_rows", "attn_q", "miss_read", "miss_write"),
    "k_combine": ("out_lse",),
}


def kernel_algorithmic_bytes(workload):
    import sys
    sys.path.insert(0, ROOT)
    import bench
    from top_sparse_attention_ls_amd import synth
    wl = synth.WORKLOADS[workload]
    n_miss = round(wl.miss_rate * wl.topk) * wl.batch if wl.hot_slots else 0
    ab = bench.algorithmic_bytes(wl, n_miss)
    return {k: sum(ab[p] for p in parts) for k, parts in KERNEL_PARTS.items()}


def _all_counters(path):
    """{(kernel short name, counter): [values in dispatch order]}"""
    out = {}
    rows = []
    for r in csv.DictReader(open(path)):
        rows.append((int(r["Dispatch_Id"]), short_name(r["Kernel_Name"]), r["Counter_Name"],
                     float(r["Counter_Value"])))
    rows.sort()
    for _, k, c, v in rows:
        out.setdefault((k, c), []).append(v)
    return out


def cmd_counters(args):
    copy_kib = args.copy_mib * 1024.0
    per = {}     # kernel -> counter -> average per launch (later half of the launches)
    launches = {}
    factors = {}
    for path in args.passes:
        vals = _all_counters(path)
        for (k, c), v in vals.items():
            if k == COPY_KERNEL or k.endswith(COPY_KERNEL):
                if c in ("FETCH_SIZE", "WRITE_SIZE") and len(v) >= 2:
                    factors[c] = copy_kib / (sum(v[-2:]) / 2)
                continue
            if not k.startswith("ls::"):
                continue
            steady = v[len(v) // 2:] if len(v) > 2 else v
            per.setdefault(k, {})[c] = sum(steady) / len(steady)
            launches[k] = max(launches.get(k, 0), len(v))
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        f = factors.get(c)
        if f is not None and not (0.4 < f < 2.6):
            raise SystemExit("%s calibration factor %.3f is implausible" % (c, f))
    alg = kernel_algorithmic_bytes(args.workload) if args.workload else {}
    res = {"workload": args.workload, "commands": args.cmd, "calibration_factors": factors,
           "kernels": {}}
    counters = sorted({c for d in per.values() for c in d})
    lines = ["# Per-kernel counters, %s" % args.workload, "",
             "Commands (one rocprofv3 --pmc pass each):", "", "```"] + args.cmd + ["```", ""]
    if factors:
        lines += ["FETCH_SIZE / WRITE_SIZE are KiB per dispatch, scaled by what each reads for a "
                  "plain %d MiB device copy in the same run (factors: %s)." % (
                      args.copy_mib, ", ".join("%s %.3f" % kv for kv in sorted(factors.items()))),
                  ""]
    hdr = ["kernel", "launches"]
    if "FETCH_SIZE" in counters and "WRITE_SIZE" in counters:
        hdr += ["HBM bytes / launch (fetch + write)", "algorithmic bytes", "ratio"]
    other = [c for c in counters if c not in ("FETCH_SIZE", "WRITE_SIZE")]
    hdr += other
    lines += ["| " + " | ".join(hdr) + " |", "|" + "---|" * len(hdr)]
    for k in sorted(per, key=lambda k: -per[k].get("FETCH_SIZE", 0)):
        d = per[k]
        base = k.split("<")[0].replace("ls::", "")
        if base == "k_attn_mfma" and k.replace(" ", "").endswith(",true>"):
            base = "k_attn_fused"  # the miss gather folded into the tile DMA
        if base == "k_coarse32":
            base = "k_coarse"  # the same pass on 32-head tiles
        if base == "k_combine_wide":
            base = "k_combine"  # the same merge, one workgroup per row
        row = ["`%s`" % k, str(launches[k])]
        entry = {"launches": launches[k], "counters": d}
        if "FETCH_SIZE" in counters and "WRITE_SIZE" in counters:
            fb = d.get("FETCH_SIZE", 0) * factors.get("FETCH_SIZE", 1.0) * 1024
            wb = d.get("WRITE_SIZE", 0) * factors.get("WRITE_SIZE", 1.0) * 1024
            a = alg.get(base)
            entry.update(fetch_bytes=round(fb), write_bytes=round(wb), algorithmic_bytes=a)
            row += ["%.3g + %.3g = %.4g" % (fb, wb, fb + wb), "%d" % a if a else "-",
                    "%.3f" % ((fb + wb) / a) if a else "-"]
        row += ["%.4g" % d[c] if c in d else "-" for c in other]
        res["kernels"][k] = entry
        lines.append("| " + " | ".join(row) + " |")
    if args.note:
        lines += ["", args.note]
    open(args.out, "w").write("\n".join(lines) + "\n")
    json.dump(res, open(os.path.splitext(args.out)[0] + ".json", "w"), indent=1)
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="action", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--out", required=True)
    s.add_argument("--cmd", required=True)
    s.add_argument("--title", default="Kernel durations")
    s.add_argument("--note", default="")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--algorithmic", type=int, default=0)
    t.add_argument("--cmd-fetch", required=True)
    t.add_argument("--cmd-write", required=True)
    c = sub.add_parser("counters")
    c.add_argument("passes", nargs="+")
    c.add_argument("--copy-mib", type=int, default=0)
    c.add_argument("--workload", default="")
    c.add_argument("--out", required=True)
    c.add_argument("--cmd", action="append", default=[])
    c.add_argument("--note", default="")
    args = ap.parse_args()
    {"stats": cmd_stats, "traffic": cmd_traffic, "counters": cmd_counters}[args.action](args)


if __name__ == "__main__":
    main()
