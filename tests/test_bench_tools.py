"""CPU checks of the measurement tooling: bench.py's single-GPU contract and counter lookup,
and bench_counters.py's parsing of rocprofv3 output (synthetic CSV files in the rocprofv3
column layout)."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import bench_counters  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout.strip()


def test_headline_is_the_long_causal_workload():
    w = bench.HEADLINE
    assert (w["B"], w["H"], w["H_kv"], w["N"], w["d"], w["causal"]) == (2, 16, 16, 8192, 128, True)
    # 4 * B * H * N^2 * d / 2
    assert bench.fwd_flops(2, 16, 8192, 8192, 128, True) == 549755813888.0


def test_source_hash_is_per_kernel_family():
    fwd = bench.kernel_source_hash("fwd_kernel<128, true>")
    assert fwd == bench.kernel_source_hash("fwd_kernel<64, false, 2>")
    dec = bench.kernel_source_hash("decode_split_kernel<128, false, false>")
    assert dec == bench.kernel_source_hash("combine_kernel<128>")
    assert fwd != dec != bench.kernel_source_hash("bwd_dq_kernel<64, true>")
    with pytest.raises(KeyError):
        bench.kernel_source_hash("mystery_kernel<1>")


def test_traffic_lookup_honours_the_hash(tmp_path, monkeypatch):
    name = "fwd_kernel<128, true> grid=262144"
    good = {"kernels": {name: {"source_hash": bench.kernel_source_hash(name), "hbm_bytes_per_launch": 123}}}
    f = tmp_path / "c.json"
    f.write_text(json.dumps(good))
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(f))
    assert bench.traffic_from_counters(name)[0] == 123
    stale = {"kernels": {name: {"source_hash": "0" * 16, "hbm_bytes_per_launch": 123}}}
    f.write_text(json.dumps(stale))
    assert bench.traffic_from_counters(name) == (None, "kernel changed since the counters were taken")
    assert bench.traffic_from_counters("fwd_kernel<64, true> grid=1")[0] is None


def test_kernel_names():
    full = "void fa::(anonymous namespace)::fwd_kernel<128, true, 0>(unsigned short const*, ...)"
    assert bench_counters.kernel_key(full) == "fwd_kernel<128, true>"
    assert bench_counters.kernel_key("fa::fwd_kernel<64, false, 4>(...)") == "fwd_kernel<64, false, 4>"
    assert bench_counters.kernel_key("decode_split_kernel<128, true, false>(...)") == "decode_split_kernel<128, true, false>"
    assert bench_counters.kernel_key("__amd_rocclr_copyBuffer") == "copy"
    assert bench_counters.kernel_key("__amd_rocclr_fillBufferAligned") is None


def write_counters(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_counters_average_per_dispatch_and_merge_runs(tmp_path):
    fk = "fwd_kernel<128, true, 0>(...)"
    dk = "decode_split_kernel<128, false, false>(...)"
    # two L2 channels per dispatch are summed; two dispatches are averaged
    rows = [dict(Dispatch_Id=1, Kernel_Name=fk, Grid_Size=262144, Counter_Name="FETCH_SIZE", Counter_Value=v)
            for v in (10, 20)] + \
           [dict(Dispatch_Id=2, Kernel_Name=fk, Grid_Size=262144, Counter_Name="FETCH_SIZE", Counter_Value=v)
            for v in (20, 30)]
    write_counters(str(tmp_path / "a"), rows + [dict(Dispatch_Id=3, Kernel_Name=dk, Grid_Size=131072,
                                                     Counter_Name="FETCH_SIZE", Counter_Value=100)])
    write_counters(str(tmp_path / "b"), rows + [dict(Dispatch_Id=3, Kernel_Name=dk, Grid_Size=131072,
                                                     Counter_Name="FETCH_SIZE", Counter_Value=900)])
    per = bench_counters.read_counter(str(tmp_path / "a"), "FETCH_SIZE", "N_k=4096")
    per = bench_counters.read_counter(str(tmp_path / "b"), "FETCH_SIZE", "N_k=65536", per)
    fetch = bench_counters.averages(per)
    assert fetch["fwd_kernel<128, true> grid=262144 N_k=4096"] == 40.0
    write = {k: 1.0 for k in fetch}
    f, w = bench_counters.merge_unchanged(dict(fetch), write, ["N_k=4096", "N_k=65536"])
    # the forward reads the same in both runs: listed once; the decode kernel differs: kept per run
    assert f["fwd_kernel<128, true> grid=262144"] == 40.0
    assert "fwd_kernel<128, true> grid=262144 N_k=4096" not in f
    assert f["decode_split_kernel<128, false, false> grid=131072 N_k=4096"] == 100.0
    assert f["decode_split_kernel<128, false, false> grid=131072 N_k=65536"] == 900.0


def test_headline_trace_reads_its_own_leg(tmp_path, monkeypatch):
    """The headline check averages the last launches of the first uninterrupted run of the
    headline kernel, not later launches of the same kernel (another leg's warm-up)."""
    d = tmp_path / "trace"
    d.mkdir()
    name = "fa::fwd_kernel<128, true, 0>(...)"
    other = "fa::fwd_kernel<64, false, 0>(...)"
    rows, t = [], 0
    for dur in [900] * 5 + [500] * 10:  # settle (slow) then the timed steps
        rows.append((name, t, t + dur)); t += dur + 10
    rows.append((other, t, t + 100)); t += 110
    for dur in [2000] * 10:  # a later leg's launches of the same kernel
        rows.append((name, t, t + dur)); t += dur + 10
    with open(d / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"])
        for n, a, b in rows:
            w.writerow([n, a, b, 262144 if "128" in n else 524288, 1, 1])
    with open(d / "run_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"])
        w.writerow([name, 25, 1000, 500, 2000, 90.0])
    text = bench_counters.trace_summary(str(d), "cmd", tail=10)
    line = [l for l in text.splitlines() if l.startswith("Headline step")][0]
    assert "averages 0.50 us over the last 10 launches" in line
    assert "15 launches" in line
