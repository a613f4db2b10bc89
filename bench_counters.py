#!/usr/bin/env python3
"""Turn two rocprofv3 counter runs into HBM bytes per kernel launch.

    cd /tmp && export TMPDIR=/tmp
    rocprofv3 --pmc FETCH_SIZE --kernel-trace --output-format csv -d OUT/fetch -o run -- \\
        python3 <repo>/bench.py --legs fwd,decode,copy --steps 3 --warmup 1 --decode-reps 3
    rocprofv3 --pmc WRITE_SIZE --kernel-trace --output-format csv -d OUT/write -o run -- \\
        python3 <repo>/bench.py --legs fwd,decode,copy --steps 3 --warmup 1 --decode-reps 3
    python3 <repo>/bench_counters.py OUT/fetch OUT/write
    # or, with several runs (decode kernels of different cache lengths share one grid):
    python3 <repo>/bench_counters.py N_k=4096=OUT/f4096,OUT/w4096 N_k=65536=OUT/f65536,OUT/w65536

FETCH_SIZE and WRITE_SIZE (KiB per dispatch, summed over the L2 channels) are scaled by
what the same counters read for the bench's plain 1 GiB device copy (`--legs copy`):
factor = known bytes / counted bytes, separately for reads and writes.  The result goes
to profiles/hbm_counters.json (read by bench.py, which reports it as roofline.traffic
only while the kernel sources still hash the same) and profiles/hbm_counters.md.
"""
from __future__ import annotations

import csv
import glob
import json
import os
import re
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

COPY_BYTES = 1024 ** 3  # bench.py leg_copy: 1 GiB read and 1 GiB written per copy


def kernel_key(name: str) -> str | None:
    m = re.search(r"(fwd_kernel<\d+, (?:true|false)>|decode_split_kernel<\d+(?:, (?:true|false))?>|combine_kernel<\d+>)",
                  name)
    if m:
        return m.group(1)
    if "copy" in name.lower() and "fill" not in name.lower():
        return "copy"
    return None


def read_counter(run_dir: str, counter: str, label: str = "", per=None) -> dict:
    """Average per dispatch of `counter`, keyed by kernel and grid (decode kernels also by label)."""
    per = per if per is not None else defaultdict(lambda: defaultdict(float))
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % run_dir)
    for f in files:
        for row in csv.DictReader(open(f)):
            if row["Counter_Name"] != counter:
                continue
            key = kernel_key(row["Kernel_Name"])
            if key:
                key += " grid=%s" % row["Grid_Size"]
                # the prefill launches are the same in every run; the rest depend on N_k
                if label and not key.startswith(("copy", "fwd_kernel<64")):
                    key += " " + label
                per[key][(f, row["Dispatch_Id"])] += float(row["Counter_Value"])
    return per


def averages(per) -> dict:
    return {k: sum(v.values()) / len(v) for k, v in per.items()}


def main():
    args = sys.argv[1:]
    if len(args) == 2 and "=" not in args[0]:
        runs = [("", args[0], args[1])]
    elif args and all("=" in a and "," in a for a in args):
        runs = []
        for a in args:
            label, dirs = a.rsplit("=", 1)
            f_dir, w_dir = dirs.split(",")
            runs.append((label, f_dir, w_dir))
    else:
        raise SystemExit(__doc__)
    import bench

    fetch_per, write_per = None, None
    for label, f_dir, w_dir in runs:
        fetch_per = read_counter(f_dir, "FETCH_SIZE", label, fetch_per)
        write_per = read_counter(w_dir, "WRITE_SIZE", label, write_per)
    fetch, write = averages(fetch_per), averages(write_per)
    # The calibration copy is the 1 GiB one: the largest copy dispatch (other, small
    # runtime copies of the bench's set-up also match the name).
    copies = [k for k in fetch if k.startswith("copy") and k in write]
    if not copies:
        raise SystemExit("the copy kernel is missing from the runs (use --legs ...,copy)")
    big = max(copies, key=lambda k: fetch[k])
    fetch["copy"], write["copy"] = fetch[big], write[big]
    f_read = COPY_BYTES / (fetch["copy"] * 1024.0)
    f_write = COPY_BYTES / (write["copy"] * 1024.0)
    kernels = {}
    for k in sorted(set(fetch) & set(write)):
        if k.startswith("copy"):
            continue
        kernels[k] = {"fetch_kib": round(fetch[k], 1), "write_kib": round(write[k], 1),
                      "hbm_read_bytes_per_launch": round(fetch[k] * 1024 * f_read),
                      "hbm_write_bytes_per_launch": round(write[k] * 1024 * f_write),
                      "hbm_bytes_per_launch": round(fetch[k] * 1024 * f_read + write[k] * 1024 * f_write)}
    out = {"kernel_source_hash": bench.kernel_source_hash(), "copy_bytes": COPY_BYTES,
           "copy_fetch_kib": round(fetch["copy"], 1), "copy_write_kib": round(write["copy"], 1),
           "factor_read": round(f_read, 4), "factor_write": round(f_write, 4), "kernels": kernels,
           "command": "rocprofv3 --pmc FETCH_SIZE|WRITE_SIZE --kernel-trace --output-format csv -- "
                      "python3 bench.py --legs fwd,decode,copy --decode-nk NK --steps 3 --warmup 1 --decode-reps 3"}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", "hbm_counters.json"), "w") as f:
        json.dump(out, f, indent=1)
    lines = ["# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE, calibrated)", "",
             "Commands (run from /tmp with TMPDIR=/tmp, one counter per run, for each cache length NK "
             "of the decode leg):", "",
             "    rocprofv3 --pmc FETCH_SIZE --kernel-trace --output-format csv -d OUT/FETCH_SIZE_NK -o run -- "
             "python3 <repo>/bench.py --legs fwd,decode,copy --decode-nk NK --steps 3 --warmup 1 --decode-reps 3",
             "    rocprofv3 --pmc WRITE_SIZE --kernel-trace --output-format csv -d OUT/WRITE_SIZE_NK -o run -- "
             "python3 <repo>/bench.py --legs fwd,decode,copy --decode-nk NK --steps 3 --warmup 1 --decode-reps 3",
             "    python3 <repo>/bench_counters.py " + " ".join(
                 "%s=OUT/FETCH_SIZE_%s,OUT/WRITE_SIZE_%s" % (lab, lab.split("=")[-1], lab.split("=")[-1])
                 if lab else "OUT/fetch OUT/write" for lab, _, _ in runs), "",
             "Calibration: the bench's 1 GiB device copy reads FETCH_SIZE %.0f KiB and WRITE_SIZE %.0f KiB, "
             "so counted reads are scaled by %.4f and writes by %.4f." % (fetch["copy"], write["copy"], f_read, f_write),
             "Kernel sources hash: `%s`." % out["kernel_source_hash"], "",
             "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB | HBM write MB |", "|---|---|---|---|---|"]
    for k, v in kernels.items():
        lines.append("| %s | %.0f | %.0f | %.2f | %.2f |" % (k, v["fetch_kib"], v["write_kib"],
                                                          v["hbm_read_bytes_per_launch"] / 1e6,
                                                          v["hbm_write_bytes_per_launch"] / 1e6))
    with open(os.path.join(ROOT, "profiles", "hbm_counters.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps(out, indent=1))


if __name__ == "__main__":
    main()
