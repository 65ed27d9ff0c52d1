"""Short text summaries of rocprofv3 runs of bench.py, for profiles/.

  python -m long_context_attention_04_amd.rocprof_summary kernels OUT_DIR SUMMARY.txt "COMMAND" [TITLE]
      per-kernel calls and durations from a --kernel-trace --stats run (--output-format csv)
  python -m long_context_attention_04_amd.rocprof_summary counters SUMMARY.txt "COMMANDS" TITLE DIR1 [DIR2 ...]
      per-kernel mean value per dispatch of every counter collected in the --pmc runs in DIR1..;
      FETCH_SIZE / WRITE_SIZE (KiB) are also scaled by what the same counter reads for the
      bench's known-size device copy (--copy-calibration), giving bytes per launch
  python -m long_context_attention_04_amd.rocprof_summary source-hash
      the hash of the headline indexer's sources that a counter summary is keyed on

Reads the CSV files rocprofv3 writes under its output directory; writes plain text.
"""
from __future__ import annotations

import csv
import glob
import os
import sys
from collections import defaultdict

COPY_KERNEL = "copyBuffer"  # the runtime's device-to-device copy kernel (the calibration copy)


def _rows(pattern_dir, suffix):
    out = []
    for path in glob.glob(os.path.join(pattern_dir, "**", f"*{suffix}"), recursive=True):
        with open(path, newline="") as f:
            out.extend(csv.DictReader(f))
    return out


def _short(name: str, n: int = 70) -> str:
    name = name.split("(")[0] if "(" in name and "<" not in name.split("(")[0] else name
    return name if len(name) <= n else name[: n - 3] + "..."


def kernels(out_dir, summary, command, title=""):
    rows = _rows(out_dir, "kernel_stats.csv")
    if not rows:
        raise SystemExit(f"no kernel_stats.csv under {out_dir}")
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    with open(summary, "w") as f:
        f.write(f"# {title}\n" if title else "")
        f.write(f"# command: {command}\n")
        f.write("# source: rocprofv3 --kernel-trace --stats (kernel_stats.csv); durations in microseconds\n")
        f.write(f"{'kernel':72s} {'calls':>7s} {'total_us':>11s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'pct':>6s}\n")
        for r in rows:
            f.write(f"{_short(r['Name']):72s} {int(r['Calls']):7d} {float(r['TotalDurationNs']) / 1e3:11.1f} "
                    f"{float(r['AverageNs']) / 1e3:9.2f} {float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} "
                    f"{float(r['Percentage']):6.1f}\n")
    print(open(summary).read())


def counters(summary, commands, title, dirs):
    vals = defaultdict(lambda: defaultdict(list))  # kernel -> counter -> per-dispatch values
    for d in dirs:
        per = defaultdict(float)  # (dispatch, kernel, counter) -> summed over instances
        for r in _rows(d, "counter_collection.csv"):
            per[(r["Dispatch_Id"], r["Kernel_Name"], r["Counter_Name"])] += float(r["Counter_Value"])
        for (_, kname, cname), v in per.items():
            vals[kname][cname].append(v)
    scale = {}
    for kname, cs in vals.items():
        if COPY_KERNEL in kname:
            for c in ("FETCH_SIZE", "WRITE_SIZE"):
                if c in cs:
                    scale[c] = cs[c]
    with open(summary, "w") as f:
        f.write(f"# {title}\n")
        for line in commands.split(";"):
            f.write(f"# command: {line.strip()}\n")
        f.write("# values: mean counter value per dispatch (instances summed)\n")
        calib = {}
        if scale:
            f.write("# FETCH_SIZE / WRITE_SIZE are KiB; bytes = KiB * 1024 * (copy bytes / the copy's own reading)\n")
        for kname in sorted(vals, key=lambda k: -len(vals[k].get("FETCH_SIZE", vals[k].get("WRITE_SIZE", [0])))):
            cs = vals[kname]
            f.write(f"kernel = {_short(kname, 120)}\n")
            for cname in sorted(cs):
                v = cs[cname]
                mean = sum(v) / len(v)
                f.write(f"  {cname} = {mean:.1f}  (dispatches {len(v)})\n")
                if cname in calib:
                    f.write(f"  {cname}_bytes_per_launch = {mean * 1024 * calib[cname]:.0f}\n")
        print(open(summary).read())


def source_hash():
    import hashlib
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
    h = hashlib.sha256()
    for f in ["index.hip", "index_fp4.h", "select.h", "common.h", "compress_block.h", "kernels.h"]:
        h.update(open(os.path.join(csrc, f), "rb").read())
    print(h.hexdigest()[:16])


if __name__ == "__main__":
    mode = sys.argv[1]
    if mode == "kernels":
        kernels(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5] if len(sys.argv) > 5 else "")
    elif mode == "counters":
        counters(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5:])
    elif mode == "source-hash":
        source_hash()
    else:
        raise SystemExit(__doc__)
