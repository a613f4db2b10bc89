#!/usr/bin/env python3
"""Turn two rocprofv3 counter runs into HBM bytes per kernel launch.

    cd /tmp && export TMPDIR=/tmp
    rocprofv3 --pmc FETCH_SIZE --kernel-trace --output-format csv -d OUT/fetch -o run -- \\
        python3 <repo>/bench.py --legs fwd,fwd_other,decode,copy --steps 3 --warmup 1 --decode-reps 3
    rocprofv3 --pmc WRITE_SIZE --kernel-trace --output-format csv -d OUT/write -o run -- \\
        python3 <repo>/bench.py --legs fwd,fwd_other,decode,copy --steps 3 --warmup 1 --decode-reps 3
    python3 <repo>/bench_counters.py OUT/fetch OUT/write
    # or, with several runs (decode kernels of different cache lengths share one grid):
    python3 <repo>/bench_counters.py N_k=4096=OUT/f4096,OUT/w4096 N_k=65536=OUT/f65536,OUT/w65536

    # shader counters (MFMA and VALU activity, LDS bank conflicts) of one run:
    rocprofv3 --pmc SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_INSTS_MFMA SQ_INSTS_VALU \
        SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_WAVE_CYCLES GRBM_GUI_ACTIVE --kernel-trace --output-format csv -d OUT/sq -o run -- \
        python3 <repo>/bench.py --legs fwd,fwd_other,bwd,fp8,decode --decode-nk 65536 --steps 3 --warmup 1 --decode-reps 3
    python3 <repo>/bench_counters.py sq OUT/sq        # -> profiles/sq_counters.md and .json
    # kernel durations of a plain bench run:
    rocprofv3 --kernel-trace --stats --output-format csv -d OUT/trace -o run -- python3 <repo>/bench.py
    python3 <repo>/bench_counters.py trace OUT/trace [N_k=4096=OUT/trace_4096 N_k=65536=OUT/trace_65536]
    #   -> profiles/kernel_trace.md (decode kernels by cache length from the labelled runs of
    #      bench.py --legs decode --decode-nk NK)

FETCH_SIZE and WRITE_SIZE (KiB per dispatch, summed over the L2 channels) are scaled by
what the same counters read for the bench's plain 1 GiB device copy (`--legs copy`):
factor = known bytes / counted bytes, separately for reads and writes.  The result goes
to profiles/hbm_counters.json (read by bench.py, which reports it as roofline.traffic
only while that kernel's sources still hash the same) and profiles/hbm_counters.md.
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


def short_name(name: str) -> str:
    """The forward's third template argument (the share of polynomial exponentials) is shown
    only when it is not 0: fwd_kernel<128, true, 0> is the plain forward fwd_kernel<128, true>."""
    return re.sub(r"(fwd_kernel<\d+, (?:true|false)), 0>", r"\1>", name)


def kernel_key(name: str) -> str | None:
    m = re.search(r"(fwd_kernel<\d+, (?:true|false)(?:, \d+)?>|decode_split_kernel<\d+(?:, (?:true|false)){0,2}>|"
                  r"combine_kernel<\d+>)", name)
    if m:
        return short_name(m.group(1))
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
                if label and not key.startswith("copy"):
                    key += " " + label
                per[key][(f, row["Dispatch_Id"])] += float(row["Counter_Value"])
    return per


def averages(per) -> dict:
    return {k: sum(v.values()) / len(v) for k, v in per.items()}


def merge_unchanged(fetch: dict, write: dict, labels: list, tol: float = 0.03):
    """Kernels whose launches read and write the same (within `tol`) in every labelled run
    (the prefill legs, which do not depend on the decode cache length) are listed once,
    without a label; the others keep one entry per run."""
    labels = [l for l in labels if l]
    if len(labels) < 2:
        return fetch, write
    bases = {k[: -len(" " + l)] for k in fetch for l in labels if k.endswith(" " + l)}
    for base in bases:
        keys = [base + " " + l for l in labels]
        if not all(k in fetch and k in write for k in keys):
            continue
        same = all(max(d[k] for k in keys) <= (1 + tol) * min(d[k] for k in keys) for d in (fetch, write))
        if same:
            for d in (fetch, write):
                d[base] = sum(d[k] for k in keys) / len(keys)
                for k in keys:
                    del d[k]
    return fetch, write


SIMDS = 256 * 4  # MI355X: 256 compute units of 4 SIMDs
XCDS = 8         # GRBM_GUI_ACTIVE is summed over the 8 XCDs (each has its own graphics block)
SQ_KERNELS = r"(fwd_kernel<\d+, (?:true|false)(?:, \d+)?>|fwd_fp8_kernel<\d+, (?:true|false)>|fp8_quant_kernel<\d+>|" \
             r"bwd_\w+<\d+(?:, (?:true|false))?>|decode_split_kernel<\d+(?:, (?:true|false)){0,2}>|combine_kernel<\d+>)"


def sq_summary(run_dir: str, cmd: str) -> str:
    """Average per dispatch of every SQ counter of a run, per kernel and grid, plus ratios:
    MFMA busy / busy cycles, VALU-active / wave cycles, LDS bank conflicts per LDS instruction."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % run_dir)
    per = defaultdict(lambda: defaultdict(lambda: defaultdict(float)))
    dur = defaultdict(dict)  # key -> {(file, dispatch): duration in ns}
    for f in files:
        for row in csv.DictReader(open(f)):
            m = re.search(SQ_KERNELS, row["Kernel_Name"])
            if m:
                key = "%s grid=%s" % (short_name(m.group(1)), row["Grid_Size"])
                per[key][row["Counter_Name"]][(f, row["Dispatch_Id"])] += float(row["Counter_Value"])
                if "End_Timestamp" in row:
                    dur[key][(f, row["Dispatch_Id"])] = int(row["End_Timestamp"]) - int(row["Start_Timestamp"])
    import bench

    names = ["SQ_BUSY_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_MFMA",
             "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "GRBM_GUI_ACTIVE"]
    lines = ["# Shader counters per kernel launch (rocprofv3 SQ counters, averages per dispatch)", "",
             "Command (from /tmp, TMPDIR=/tmp):", "", "    " + cmd, "    python3 <repo>/bench_counters.py sq OUT/sq", "",
             "GPU cycles = GRBM_GUI_ACTIVE / %d XCDs (the launch's duration in cycles); MFMA busy %% = "
             "SQ_VALU_MFMA_BUSY_CYCLES / (GPU cycles x %d SIMDs); VALU active %% = "
             "SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES (the waves' share of cycles issuing VALU); conflicts / LDS instr = "
             "SQ_LDS_BANK_CONFLICT / SQ_INSTS_LDS; clock = GPU cycles / the dispatch's duration in the same run "
             "(profiled launches run longer than plain ones); MFMA busy at 2.4 GHz = MFMA busy %% x clock / 2.4 GHz, "
             "the share of the nominal-clock peak the matrix cores delivered." % (XCDS, SIMDS), "",
             "| kernel | GPU cycles | clock GHz | MFMA busy % | MFMA busy at 2.4 GHz % | VALU active % | MFMA instr | VALU instr | LDS instr | LDS bank conflicts | conflicts / LDS instr |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    table = {}
    for key in sorted(per):
        avg = {n: (sum(per[key][n].values()) / len(per[key][n])) if per[key][n] else float("nan") for n in names}
        gpu = avg["GRBM_GUI_ACTIVE"] / XCDS
        clocks = [per[key]["GRBM_GUI_ACTIVE"][d] / XCDS / ns for d, ns in dur[key].items()
                  if ns > 0 and d in per[key]["GRBM_GUI_ACTIVE"]]
        ghz = sum(clocks) / len(clocks) if clocks else float("nan")
        busy = 100.0 * avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (gpu * SIMDS) if gpu else float("nan")
        table[key] = {"source_hash": bench.kernel_source_hash(key), "gpu_cycles": round(gpu),
                      "clock_ghz": round(ghz, 3) if clocks else None, "mfma_busy_pct": round(100.0 * avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (gpu * SIMDS), 2)
                      if gpu else None, "lds_instr": round(avg["SQ_INSTS_LDS"]),
                      "lds_bank_conflicts": round(avg["SQ_LDS_BANK_CONFLICT"])}
        lines.append("| %s | %.0f | %.2f | %.1f | %.1f | %.1f | %.0f | %.0f | %.0f | %.0f | %.4f |" % (
            key, gpu, ghz, busy, busy * ghz / 2.4,
            100.0 * avg["SQ_ACTIVE_INST_VALU"] / avg["SQ_WAVE_CYCLES"] if avg["SQ_WAVE_CYCLES"] else float("nan"),
            avg["SQ_INSTS_MFMA"], avg["SQ_INSTS_VALU"], avg["SQ_INSTS_LDS"], avg["SQ_LDS_BANK_CONFLICT"],
            avg["SQ_LDS_BANK_CONFLICT"] / avg["SQ_INSTS_LDS"] if avg["SQ_INSTS_LDS"] else float("nan")))
    return "\n".join(lines) + "\n", table


def trace_summary(run_dir: str, cmd: str, tail: int = 200) -> str:
    """Markdown summary of a rocprofv3 --kernel-trace --stats run (csv): per-kernel statistics
    and per-launch-shape averages (the last `tail` calls of a shape are the bench's
    back-to-back loop, after its warm-up)."""
    stats = list(csv.DictReader(open(os.path.join(run_dir, "run_kernel_stats.csv"))))
    trace = sorted(csv.DictReader(open(os.path.join(run_dir, "run_kernel_trace.csv"))),
                   key=lambda r: int(r["Start_Timestamp"]))

    def short(n):
        m = re.search(SQ_KERNELS, n)
        return short_name(m.group(1)) if m else n.split("(")[0][:60]

    out = ["# Kernel trace of a bench.py run (all legs but the CPU baseline)", "",
           "Command (from /tmp, TMPDIR=/tmp):", "", "    " + cmd, "    python3 <repo>/bench_counters.py trace OUT/trace", "",
           "| kernel | calls | average us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in stats:
        out.append("| %s | %s | %.2f | %.2f | %.2f | %.1f |" % (short(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3,
                                                             float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
                                                             float(r["Percentage"])))
    g = defaultdict(list)
    for r in trace:
        key = "%s grid=%s" % (short(r["Kernel_Name"]), int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]))
        g[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out += ["", "Per launch shape (grid = work-items); the last column averages the last %d calls of the shape." % tail,
            "", "| kernel, grid | calls | average us | min us | last %d average us |" % tail, "|---|---|---|---|---|"]
    for k, v in sorted(g.items()):
        if not re.search(SQ_KERNELS, k):
            continue
        out.append("| %s | %d | %.2f | %.2f | %.2f |" % (k, len(v), sum(v) / len(v), min(v), sum(v[-tail:]) / len(v[-tail:])))
    # the headline step's kernel: its rate from this trace, to compare with bench.py's roofline line
    import bench

    w = bench.HEADLINE
    t_r = -(-w["N"] // 128)
    grid = ((t_r + 1) // 2 if w["causal"] else t_r) * w["B"] * w["H"] * 256
    key = "fwd_kernel<%d, %s> grid=%d" % (w["d"], "true" if w["causal"] else "false", grid)
    if key in g:
        # the headline leg runs first and launches only this kernel: its timed steps are the
        # last `tail` launches of the first uninterrupted run of the kernel in the trace
        run, started = [], False
        for r in trace:
            k = "%s grid=%s" % (short(r["Kernel_Name"]),
                                int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]))
            if k == key:
                started = True
                run.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
            elif started:
                break
        v = run[-tail:]
        us = sum(v) / len(v)
        fl = bench.fwd_flops(w["B"], w["H"], w["N"], w["N"], w["d"], w["causal"])
        out += ["", "Headline step (%s): %s averages %.2f us over the last %d launches of its leg (the first "
                "uninterrupted run of the kernel, %d launches with the clock settle and warm-up), so %.1f TFLOP/s "
                "= %.4f of the %.1f TFLOP/s bf16 peak (bench.py's roofline.frac comes from HIP events around the "
                "same launches)." % (w["name"], key, us, len(v), len(run), fl / us / 1e6,
                                     fl / us / 1e6 / bench.PEAK_BF16_TFLOPS, bench.PEAK_BF16_TFLOPS)]
    return "\n".join(out) + "\n"


def decode_trace_summary(labelled: list) -> str:
    """Decode kernels of one kernel-trace run per cache length (their launches share one grid
    across cache lengths, so a single run cannot tell them apart)."""
    out = ["", "Decode kernels by cache length (one run per length):", "",
           "    rocprofv3 --kernel-trace --stats --output-format csv -d OUT/trace_NK -o run -- "
           "python3 <repo>/bench.py --legs decode --decode-nk NK", "",
           "| cache length | kernel | calls | median us | average us | min us |", "|---|---|---|---|---|---|"]
    for label, run_dir in labelled:
        g = defaultdict(list)
        for r in csv.DictReader(open(os.path.join(run_dir, "run_kernel_trace.csv"))):
            m = re.search(r"(decode_split_kernel<\d+(?:, (?:true|false)){1,2}>|combine_kernel<\d+>)", r["Kernel_Name"])
            if m:
                g[m.group(1)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        for k, v in sorted(g.items()):
            v = sorted(v)
            out.append("| %s | %s | %d | %.2f | %.2f | %.2f |" % (label, k, len(v), v[len(v) // 2], sum(v) / len(v), v[0]))
    out += ["", "The contiguous split kernel's median is its back-to-back launches over rotated cache copies "
            "(most of its launches); `decode_split_kernel<128, true, false>` is the paged cache and "
            "`decode_split_kernel<128, false, true>` the one-launch split and merge (`fa_decode`)."]
    return "\n".join(out) + "\n"


def main():
    args = sys.argv[1:]
    if len(args) >= 2 and args[0] == "trace":
        cmd = "rocprofv3 --kernel-trace --stats --output-format csv -d OUT/trace -o run -- python3 <repo>/bench.py"
        text = trace_summary(args[1], cmd)
        labelled = [a.split("=", 2)[1:] for a in args[2:]]  # N_k=4096=OUT/trace_4096
        if labelled:
            text += decode_trace_summary([("N_k=" + l, d) for l, d in labelled])
        with open(os.path.join(ROOT, "profiles", "kernel_trace.md"), "w") as f:
            f.write(text)
        print(text)
        return
    if len(args) == 2 and args[0] == "sq":
        cmd = ("rocprofv3 --pmc SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_INSTS_MFMA SQ_INSTS_VALU "
               "SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_WAVE_CYCLES GRBM_GUI_ACTIVE --kernel-trace --output-format csv -d OUT/sq -o run -- "
               "python3 <repo>/bench.py --legs fwd,fwd_other,bwd,fp8,decode --decode-nk 65536 --steps 3 --warmup 1 --decode-reps 3")
        text, table = sq_summary(args[1], cmd)
        with open(os.path.join(ROOT, "profiles", "sq_counters.md"), "w") as f:
            f.write(text)
        with open(os.path.join(ROOT, "profiles", "sq_counters.json"), "w") as f:
            json.dump({"command": cmd, "kernels": table}, f, indent=1)
        print(text)
        return
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
    fetch, write = merge_unchanged(averages(fetch_per), averages(write_per), [lab for lab, _, _ in runs])
    # The calibration copy is the 1 GiB one.  Other copies of the bench's set-up (the decode
    # leg's rotated cache copies, at most 537 MB each, share the copy kernel's grid; torch
    # copy kernels also match the name) are smaller, so the calibration takes the copy
    # dispatches within 1% of the largest one, per counter.
    def largest_copies(per) -> float:
        vals = [x for k, v in per.items() if k.startswith("copy") for x in v.values()]
        if not vals:
            raise SystemExit("the copy kernel is missing from the runs (use --legs ...,copy)")
        top = [x for x in vals if x >= 0.99 * max(vals)]
        return sum(top) / len(top)

    fetch["copy"], write["copy"] = largest_copies(fetch_per), largest_copies(write_per)
    f_read = COPY_BYTES / (fetch["copy"] * 1024.0)
    f_write = COPY_BYTES / (write["copy"] * 1024.0)
    kernels = {}
    for k in sorted(set(fetch) & set(write)):
        if k.startswith("copy"):
            continue
        kernels[k] = {"source_hash": bench.kernel_source_hash(k), "fetch_kib": round(fetch[k], 1), "write_kib": round(write[k], 1),
                      "hbm_read_bytes_per_launch": round(fetch[k] * 1024 * f_read),
                      "hbm_write_bytes_per_launch": round(write[k] * 1024 * f_write),
                      "hbm_bytes_per_launch": round(fetch[k] * 1024 * f_read + write[k] * 1024 * f_write)}
    out = {"copy_bytes": COPY_BYTES,
           "copy_fetch_kib": round(fetch["copy"], 1), "copy_write_kib": round(write["copy"], 1),
           "factor_read": round(f_read, 4), "factor_write": round(f_write, 4), "kernels": kernels,
           "command": "rocprofv3 --pmc FETCH_SIZE|WRITE_SIZE --kernel-trace --output-format csv -- "
                      "python3 bench.py --legs fwd,fwd_other,decode,copy --decode-nk NK --steps 3 --warmup 1 --decode-reps 3"}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", "hbm_counters.json"), "w") as f:
        json.dump(out, f, indent=1)
    lines = ["# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE, calibrated)", "",
             "Commands (run from /tmp with TMPDIR=/tmp, one counter per run, for each cache length NK "
             "of the decode leg):", "",
             "    rocprofv3 --pmc FETCH_SIZE --kernel-trace --output-format csv -d OUT/FETCH_SIZE_NK -o run -- "
             "python3 <repo>/bench.py --legs fwd,fwd_other,decode,copy --decode-nk NK --steps 3 --warmup 1 --decode-reps 3",
             "    rocprofv3 --pmc WRITE_SIZE --kernel-trace --output-format csv -d OUT/WRITE_SIZE_NK -o run -- "
             "python3 <repo>/bench.py --legs fwd,fwd_other,decode,copy --decode-nk NK --steps 3 --warmup 1 --decode-reps 3",
             "    python3 <repo>/bench_counters.py " + " ".join(
                 "%s=OUT/FETCH_SIZE_%s,OUT/WRITE_SIZE_%s" % (lab, lab.split("=")[-1], lab.split("=")[-1])
                 if lab else "OUT/fetch OUT/write" for lab, _, _ in runs), "",
             "Calibration: the bench's 1 GiB device copy reads FETCH_SIZE %.0f KiB and WRITE_SIZE %.0f KiB, "
             "so counted reads are scaled by %.4f and writes by %.4f." % (fetch["copy"], write["copy"], f_read, f_write),
             "Each kernel's entry in hbm_counters.json carries the hash of the sources it is built from; "
             "bench.py reports its traffic only while they hash the same.", "",
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
