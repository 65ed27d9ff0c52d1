"""Short text summaries of rocprofv3 runs of bench.py, for profiles/.

  python -m long_context_attention_04_amd.rocprof_summary kernels OUT_DIR SUMMARY.txt "COMMAND" [TITLE]
      per-kernel calls and durations from a --kernel-trace --stats run (--output-format csv)
  python -m long_context_attention_04_amd.rocprof_summary counters SUMMARY.txt "CMD1; CMD2" TITLE DIR1 [DIR2 ...]
          [--copy-bytes N --kernel SUBSTR --keyed]
      per-kernel mean value per dispatch of every counter collected in the --pmc runs in DIR1..;
      FETCH_SIZE / WRITE_SIZE (KiB) are also scaled by what the same counter reads for the
      bench's known-size calibration kernel (--copy-calibration: N bytes read and written),
      giving bytes per launch; --kernel adds the named kernel's fetch/write bytes per launch;
      --durations KT_DIR adds each kernel's MFMA busy fraction from the kernel trace's average duration
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

CLOCK_GHZ, SIMDS = 2.4, 1024  # MI355X: 256 CUs x 4 SIMDs at 2.4 GHz
CALIB_KERNEL = "neg_kernel"  # bench.py --copy-calibration: torch.neg over a known size
# the headline indexer's sources (bench.py keys its counter summary on the same list)
INDEX_SOURCES = ["index.hip", "index_fp4.h", "select.h", "common.h", "compress_block.h", "kernels.h"]


def _rows(pattern_dir, suffix):
    out = []
    for path in glob.glob(os.path.join(pattern_dir, "**", f"*{suffix}"), recursive=True):
        with open(path, newline="") as f:
            out.extend(csv.DictReader(f))
    return out


def _short(name: str, n: int = 70) -> str:
    """A kernel's name without its parameter list, return type and anonymous namespaces."""
    name = name.replace("(anonymous namespace)::", "").strip()
    if name.endswith(")"):  # cut the trailing parameter list
        depth = 0
        for i in range(len(name) - 1, -1, -1):
            depth += {")": 1, "(": -1}.get(name[i], 0)
            if depth == 0:
                name = name[:i]
                break
    if name.startswith("void "):
        name = name[5:]
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


def counters(summary, commands, title, dirs, copy_bytes=0, kernel=None, keyed=False, durations=None):
    vals = defaultdict(lambda: defaultdict(list))  # kernel -> counter -> per-dispatch values
    for d in dirs:
        per = defaultdict(float)  # (dispatch, kernel, counter) -> summed over instances
        for r in _rows(d, "counter_collection.csv"):
            per[(r["Dispatch_Id"], r["Kernel_Name"], r["Counter_Name"])] += float(r["Counter_Value"])
        for (_, kname, cname), v in per.items():
            vals[kname][cname].append(v)
    # bytes per KiB the counter reports, from the calibration kernel (reads and writes copy_bytes)
    calib = {}
    for kname, cs in vals.items():
        if CALIB_KERNEL in kname and copy_bytes:
            for c in ("FETCH_SIZE", "WRITE_SIZE"):
                if c in cs and cs[c][0] > 0:
                    calib[c] = copy_bytes / (cs[c][0] * 1024.0)
    lines = [f"# {title}"]
    lines += [f"# command: {c.strip()}" for c in commands.split(";") if c.strip()]
    lines.append("# values: mean counter value per dispatch (instances summed)")
    if calib:
        lines.append(f"# FETCH_SIZE / WRITE_SIZE are KiB; bytes = KiB * 1024 * factor, the factor making the "
                     f"calibration kernel ({CALIB_KERNEL}, {copy_bytes} bytes read and written) read exactly that")
        for c, f in sorted(calib.items()):
            lines.append(f"calibration_factor_{c} = {f:.4f}")
    if durations:
        lines.append(f"# derived: MFMA busy fraction = SQ_VALU_MFMA_BUSY_CYCLES / (average duration from {durations}"
                     f" x {CLOCK_GHZ} GHz x {SIMDS} SIMDs)")
    avg_ns = {}
    if durations:
        for r in _rows(durations, "kernel_stats.csv"):
            avg_ns[r["Name"]] = float(r["AverageNs"])
    main = None
    for kname in sorted(vals, key=lambda k: -max(len(v) for v in vals[k].values())):
        cs = vals[kname]
        if "csa::" not in kname and CALIB_KERNEL not in kname:
            continue  # the harness's own kernels (fills, casts, copies)
        lines.append(f"kernel: {_short(kname, 150)}")
        if kname in avg_ns and "SQ_VALU_MFMA_BUSY_CYCLES" in cs:
            busy = sum(cs["SQ_VALU_MFMA_BUSY_CYCLES"]) / len(cs["SQ_VALU_MFMA_BUSY_CYCLES"])
            lines.append(f"  average duration us: {avg_ns[kname] / 1e3:.2f}")
            lines.append(f"  MFMA busy fraction: {busy / (avg_ns[kname] * CLOCK_GHZ * SIMDS):.4f}")
        for cname in sorted(cs):
            v = cs[cname]
            mean = sum(v) / len(v)
            lines.append(f"  {cname}: {mean:.1f}  (dispatches {len(v)})")
            if cname in calib:
                lines.append(f"  {cname} bytes per launch: {mean * 1024 * calib[cname]:.0f}")
        if kernel and kernel in kname:
            main = cs
    if kernel:
        if main is None:
            raise SystemExit(f"no dispatches of {kernel}")
        lines.append(f"# the dominant kernel ({kernel}), HBM bytes per launch")
        if keyed:
            lines.append(f"source_sha256_16 = {source_hash(quiet=True)}")
        for c, key in (("FETCH_SIZE", "fetch_bytes_per_launch"), ("WRITE_SIZE", "write_bytes_per_launch")):
            if c in main and c in calib:
                lines.append(f"{key} = {sum(main[c]) / len(main[c]) * 1024 * calib[c]:.0f}")
    with open(summary, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def source_hash(quiet=False):
    import hashlib
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
    h = hashlib.sha256()
    for f in INDEX_SOURCES:
        h.update(open(os.path.join(csrc, f), "rb").read())
    if not quiet:
        print(h.hexdigest()[:16])
    return h.hexdigest()[:16]


if __name__ == "__main__":
    mode = sys.argv[1]
    if mode == "kernels":
        kernels(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5] if len(sys.argv) > 5 else "")
    elif mode == "counters":
        import argparse
        ap = argparse.ArgumentParser(prog="rocprof_summary counters")
        ap.add_argument("summary")
        ap.add_argument("commands")
        ap.add_argument("title")
        ap.add_argument("dirs", nargs="+")
        ap.add_argument("--copy-bytes", type=int, default=0)
        ap.add_argument("--kernel", default=None, help="substring naming the dominant kernel")
        ap.add_argument("--keyed", action="store_true", help="record the indexer source hash")
        ap.add_argument("--durations", default=None, help="a --kernel-trace --stats run of the same command")
        a = ap.parse_args(sys.argv[2:])
        counters(a.summary, a.commands, a.title, a.dirs, a.copy_bytes, a.kernel, a.keyed, a.durations)
    elif mode == "source-hash":
        source_hash()
    else:
        raise SystemExit(__doc__)
