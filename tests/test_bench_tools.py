"""CPU checks of bench.py's profile tooling on fabricated rocprofv3 CSVs: the verify dispatches
are told apart from a compact-cache decode of the same kernel instance (same grid, smaller
read) and matched between the two counter runs by launch order; the copy calibration scales
the counters; the kernel-trace summary averages only the timed steps' verify calls and the
merges that follow them; and a summary is trusted only for its own workload."""

import csv
import os

import bench
from kv_sparse_speculative_amd.workloads import WORKLOADS

WL = WORKLOADS["llama8b_ctx8k"]
KERNEL = bench.verify_kernel_name(WL)


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=header)
        w.writeheader()
        w.writerows(rows)


def _counters(directory, counter, values):
    header = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"]
    rows = [{"Dispatch_Id": i + 1, "Grid_Size": g, "Kernel_Name": k, "Counter_Name": counter,
             "Counter_Value": v} for i, (g, k, v) in enumerate(values)]
    _write(os.path.join(directory, "run", "x_counter_collection.csv"), header, rows)


def test_pmc_summary_picks_the_verify_dispatches(tmp_path):
    algo = bench.verify_algorithmic_bytes(WL)
    fetch_kib = algo / 2 / 1024            # FETCH_SIZE counts half the bytes (copy scale 2.0)
    copy = bench.COPY_BYTES / 1024
    # verify, compact decode (same kernel instance and grid, small read), verify, a copy, verify
    _counters(str(tmp_path / "f"), "FETCH_SIZE", [
        (65536, KERNEL, fetch_kib), (65536, KERNEL, fetch_kib / 16), (65536, KERNEL, fetch_kib),
        (512, "__amd_rocclr_copyBuffer", copy / 2), (65536, KERNEL, fetch_kib)])
    _counters(str(tmp_path / "w"), "WRITE_SIZE", [
        (65536, KERNEL, 100.0), (65536, KERNEL, 7.0), (65536, KERNEL, 100.0),
        (512, "__amd_rocclr_copyBuffer", copy), (65536, KERNEL, 100.0)])
    out = tmp_path / "summary.md"
    bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), str(out), ["cmd"], WL)
    fields = {}
    for line in open(out):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            fields[k.strip()] = v.strip()
    assert fields["FETCH_SIZE per dispatch (KiB, mean of 3)"] == f"{fetch_kib:.1f}"
    assert fields["WRITE_SIZE per dispatch (KiB, mean of 3)"] == "100.0"
    assert int(fields["HBM bytes per launch"]) == int(algo + 100 * 1024)
    assert fields["algorithmic bytes per launch"] == str(algo)


def test_trace_summary_averages_the_timed_verify_calls(tmp_path):
    header = ["Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    rows, t = [], 0
    for step in range(5):                                 # 2 warm-up + 3 timed steps
        dur = 260_000 if step < 2 else 200_000            # ns: warm-up calls a little slower
        rows.append({"Kernel_Name": f"void {KERNEL}(AttnArgs)", "Start_Timestamp": t,
                     "End_Timestamp": t + dur})
        t += dur
        rows.append({"Kernel_Name": "merge_kernel(float const*, int, int, float*, float*)",
                     "Start_Timestamp": t, "End_Timestamp": t + 10_000})
        t += 20_000
        rows.append({"Kernel_Name": f"void {KERNEL}(AttnArgs)", "Start_Timestamp": t,
                     "End_Timestamp": t + 20_000})        # a short compact-cache decode
        t += 30_000
    _write(str(tmp_path / "p" / "run_kernel_trace.csv"), header, rows)
    attn, merge = bench.verify_dispatches(str(tmp_path / "p"), WL, warmup=2)
    assert attn == [200.0, 200.0, 200.0]
    assert merge == [10.0, 10.0, 10.0]


def test_committed_traffic_is_per_workload():
    # a workload with no committed counter summary reports no traffic
    assert bench.committed_traffic("tiny_fp32") is None
    assert bench.traffic_summary_path("llama8b_ctx32k").endswith(
        os.path.join("profiles", "verify_attn_llama8b_ctx32k_traffic.md"))
