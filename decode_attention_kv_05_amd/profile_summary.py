"""Turn rocprofv3 CSV output into the short text summaries kept under profiles/.

    python -m decode_attention_kv_05_amd.profile_summary stats DIR --workload W --command "..."
        [--name STEM]
    python -m decode_attention_kv_05_amd.profile_summary traffic --workload W --nsplit N \
        --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR --copy-bytes BYTES --command "..."
        [--name STEM] [--kernel SUBSTRING] [--tag KEY] [--dispatches-per-step N]
    python -m decode_attention_kv_05_amd.profile_summary counters DIR [DIR ...] --kernel SUBSTRING \
        --name STEM --command "..."

`stats` reads a `rocprofv3 --kernel-trace --stats --output-format csv` run and
writes profiles/<STEM>_kernels.txt (STEM defaults to longflow_decode_<W>).
`traffic` reads four `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs
(the benchmark and a plain device copy of a known size, run with `bench.py
--copy-probe`), scales the per-dispatch KiB of the kernel whose name contains
SUBSTRING (default: the decode kernel) by bytes-copied / KiB-counted of the
copy and by the kernel's dispatches per decode call (--dispatches-per-step,
default 1), and writes profiles/<STEM>_traffic.txt plus the entry KEY (default
<W>/nsplit<N>) of profiles/traffic.json, tagged with the hash of the kernel
sources it measured (bench.py reports the figure only while that hash
matches).
"""

import argparse
import csv
import glob
import json
import os
import time

from .build import source_hash

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")
DECODE = "longflow_decode_kernel"
COPY_HINTS = ("copy",)


def _find(directory, suffix):
    hits = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {directory}")
    return hits[0]


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def counter_means(directory, counter):
    """Mean per-dispatch value of `counter` by kernel name."""
    sums, counts = {}, {}
    for row in _rows(_find(directory, "counter_collection.csv")):
        if row.get("Counter_Name") != counter:
            continue
        name = row["Kernel_Name"]
        sums[name] = sums.get(name, 0.0) + float(row["Counter_Value"])
        counts[name] = counts.get(name, 0) + 1
    return {k: (sums[k] / counts[k], counts[k]) for k in sums}


def _pick(means, want):
    for name, val in means.items():
        if want(name):
            return name, val
    raise KeyError(f"kernel not found among {list(means)}")


def dispatch_durations(directory):
    """Per-dispatch durations (ns) by kernel name, in dispatch order."""
    out = {}
    for row in _rows(_find(directory, "kernel_trace.csv")):
        out.setdefault(row["Kernel_Name"], []).append(int(row["End_Timestamp"]) - int(row["Start_Timestamp"]))
    return out


def _family(args):
    text = f"{args.name or ''} {getattr(args, 'kernel', None) or ''}"
    for fam in ("topk", "stack"):
        if fam in text:
            return fam
    return "decode"


def write_stats(args):
    rows = _rows(_find(args.dir, "kernel_stats.csv"))
    try:
        trace = dispatch_durations(args.dir)
    except FileNotFoundError:
        trace = {}
    out = os.path.join(PROFILES, f"{args.name or 'longflow_decode_' + args.workload}_kernels.txt")
    with open(out, "w") as f:
        f.write(f"# rocprofv3 kernel statistics, workload {args.workload}\n")
        f.write(f"# command: {args.command}\n")
        f.write(f"# kernel sources ({_family(args)}): {source_hash(_family(args))}  date: {time.strftime('%Y-%m-%d')}\n")
        f.write("# avg/min/max over every dispatch (warm-up included); p50 = median dispatch from the kernel trace\n")
        f.write(f"{'calls':>6} {'avg_us':>10} {'p50_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}  kernel\n")
        for r in rows:
            d = sorted(trace.get(r["Name"], []))
            p50 = d[len(d) // 2] / 1e3 if d else float("nan")
            f.write(f"{int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>10.2f} {p50:>10.2f} "
                    f"{float(r['MinNs']) / 1e3:>10.2f} {float(r['MaxNs']) / 1e3:>10.2f} "
                    f"{float(r['Percentage']):>6.2f}  {r['Name'][:110]}\n")
    print(out)


def write_traffic(args):
    fetch = counter_means(args.fetch, "FETCH_SIZE")
    write = counter_means(args.write, "WRITE_SIZE")
    cfetch = counter_means(args.copy_fetch, "FETCH_SIZE")
    cwrite = counter_means(args.copy_write, "WRITE_SIZE")
    want = args.kernel or DECODE
    is_decode = lambda n: want in n
    is_copy = lambda n: any(h in n.lower() for h in COPY_HINTS) and want not in n
    kname, (f_kib, nf) = _pick(fetch, is_decode)
    _, (w_kib, nw) = _pick(write, is_decode)
    cname, (cf_kib, _) = _pick(cfetch, is_copy)
    _, (cw_kib, _) = _pick(cwrite, is_copy)
    f_scale = args.copy_bytes / (cf_kib * 1024.0)
    w_scale = args.copy_bytes / (cw_kib * 1024.0)
    per_step = args.dispatches_per_step
    read_b = f_kib * 1024.0 * f_scale * per_step
    write_b = w_kib * 1024.0 * w_scale * per_step
    total = read_b + write_b
    tag = args.tag or f"{args.workload}/nsplit{args.nsplit}"
    out = os.path.join(PROFILES, f"{args.name or 'longflow_decode_' + args.workload}_traffic.txt")
    with open(out, "w") as f:
        f.write(f"# HBM traffic of {kname[:80]} from rocprofv3 counters, workload {args.workload}, "
                f"nsplit {args.nsplit}, key {tag}\n")
        f.write(f"# commands: {args.command}\n")
        f.write(f"# kernel sources ({_family(args)}): {source_hash(_family(args))}  date: {time.strftime('%Y-%m-%d')}\n")
        f.write(f"FETCH_SIZE KiB/dispatch (mean of {nf}): {f_kib:.1f}\n")
        f.write(f"WRITE_SIZE KiB/dispatch (mean of {nw}): {w_kib:.1f}\n")
        f.write(f"copy probe {cname[:60]}: {args.copy_bytes} bytes; FETCH_SIZE {cf_kib:.1f} KiB, WRITE_SIZE {cw_kib:.1f} KiB\n")
        f.write(f"scale factors (bytes per counted byte): fetch {f_scale:.4f}, write {w_scale:.4f}\n")
        if per_step != 1:
            f.write(f"dispatches of the kernel per decode call: {per_step}\n")
        f.write(f"HBM bytes per launch: read {read_b:.0f}, write {write_b:.0f}, total {total:.0f}\n")
    path = os.path.join(PROFILES, "traffic.json")
    try:
        with open(path) as f:
            db = json.load(f)
    except (OSError, ValueError):
        db = {}
    db[tag] = {"kernel_hash": source_hash(_family(args)), "bytes_per_launch": round(total), "read_bytes": round(read_b),
               "write_bytes": round(write_b), "fetch_scale": round(f_scale, 5), "write_scale": round(w_scale, 5)}
    with open(path, "w") as f:
        json.dump(db, f, indent=1, sort_keys=True)
        f.write("\n")
    print(out)


def write_counters(args):
    """Mean per-dispatch value of every counter found in the given --pmc runs,
    for the kernel whose name contains --kernel, plus a few ratios."""
    vals = {}
    kname = None
    for d in args.dirs:
        for row in _rows(_find(d, "counter_collection.csv")):
            if args.kernel not in row["Kernel_Name"]:
                continue
            kname = row["Kernel_Name"]
            vals.setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
    if not vals:
        raise KeyError(f"no counters for a kernel matching {args.kernel!r}")
    mean = {k: sum(v) / len(v) for k, v in vals.items()}
    out = os.path.join(PROFILES, f"{args.name}_counters.txt")
    with open(out, "w") as f:
        f.write(f"# rocprofv3 hardware counters of {kname[:90]}\n")
        f.write(f"# command: {args.command}\n")
        f.write(f"# kernel sources ({_family(args)}): {source_hash(_family(args))}  date: {time.strftime('%Y-%m-%d')}\n")
        f.write("# mean per dispatch over all dispatches of the kernel (summed over the device)\n")
        for k in sorted(mean):
            f.write(f"{k:28s} {mean[k]:18.1f}   ({len(vals[k])} dispatches)\n")
        ratios = [
            ("LDS bank-conflict cycles / LDS active cycles", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE"),
            ("LDS address-conflict cycles / LDS active cycles", "SQ_LDS_ADDR_CONFLICT", "SQ_LDS_IDX_ACTIVE"),
            ("LDS instructions per VALU instruction", "SQ_INSTS_LDS", "SQ_INSTS_VALU"),
            ("VALU instructions per wave", "SQ_INSTS_VALU", "SQ_WAVES"),
            ("vector-memory read instructions per wave", "SQ_INSTS_VMEM_RD", "SQ_WAVES"),
            ("VALU-active cycles / wave cycles", "SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES"),
            ("LDS-wait cycles / wave cycles", "SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES"),
        ]
        f.write("# ratios\n")
        for label, a, b in ratios:
            if a in mean and b in mean and mean[b]:
                f.write(f"{label:52s} {mean[a] / mean[b]:10.4f}\n")
    print(out)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--workload", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--name", default=None)
    t = sub.add_parser("traffic")
    for k in ("workload", "fetch", "write", "copy_fetch", "copy_write", "command"):
        t.add_argument("--" + k.replace("_", "-"), required=True)
    t.add_argument("--nsplit", type=int, required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--name", default=None)
    t.add_argument("--kernel", default=None)
    t.add_argument("--tag", default=None)
    t.add_argument("--dispatches-per-step", type=int, default=1,
                   help="dispatches of the kernel per decode call; the record is per call")
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--kernel", required=True)
    c.add_argument("--name", required=True)
    c.add_argument("--command", required=True)
    args = ap.parse_args()
    {"stats": write_stats, "traffic": write_traffic, "counters": write_counters}[args.cmd](args)


if __name__ == "__main__":
    main()
