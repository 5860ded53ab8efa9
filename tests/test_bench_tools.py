"""CPU checks of bench.py's profile tooling on fabricated rocprofv3 CSVs: a marked counter run is
split into calls at the marker kernel (kernels outside the library and the set-up segment are
dropped, repeated calls are averaged, a marker-count mismatch is an error); the copy
calibration scales the byte counters; the kernel-trace summary averages only the timed steps'
verify calls and the merges that follow them; and a summary is trusted only for its own
workload."""

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


def _marked_run(directory, counter, seq):
    """seq: list of (kernel name, value) in launch order; Dispatch_Id follows the order."""
    _counters(directory, counter, [(256, k, v) for k, v in seq])


def test_call_summary_splits_at_markers_and_scales_by_the_copy(tmp_path):
    mark = "kvss::(anonymous namespace)::philox_kernel(HIP_vector_type<unsigned int, 4u> const*)"
    rs = "void kvss::(anonymous namespace)::snap_rowstats_mfma<128, 8, false>(kvss::SnapArgs)"
    cs = "void kvss::(anonymous namespace)::snap_colscore_mfma<128, 8>(kvss::SnapArgs)"
    vk = f"void kvss::(anonymous namespace)::{KERNEL}(kvss::AttnArgs)"
    mg = "kvss::(anonymous namespace)::merge_kernel(float const*, int, int, float*, float*)"
    copy = "__amd_rocclr_copyBuffer"
    calls = ["snapkv_select", "verify", "snapkv_select", "verify", "setup", "kv_append"]
    fetch = [(mark, 0.0), (rs, 100.0), (cs, 100.0), (mark, 0.0), (vk, 400.0), (mg, 4.0),
             (mark, 0.0), (rs, 110.0), (cs, 90.0), (mark, 0.0), (vk, 400.0), (mg, 4.0),
             (mark, 0.0), ("void at::native::index_kernel(int)", 9.0), (mark, 0.0),
             ("kvss::(anonymous namespace)::kv_append_kernel(kvss::AppendArgs)", 3.0),
             (copy, bench.COPY_BYTES / 1024 / 2)]        # FETCH_SIZE reads half a copy
    write = [(k, 1.0 if k != copy else bench.COPY_BYTES / 1024) for k, _ in fetch]
    _marked_run(str(tmp_path / "f"), "FETCH_SIZE", fetch)
    _marked_run(str(tmp_path / "w"), "WRITE_SIZE", write)
    meta = tmp_path / "calls.json"
    import json
    json.dump(calls, open(meta, "w"))
    algo = {"snapkv_select": 200 * 2 * 1024, "verify": 808 * 1024, "kv_append": 6 * 1024}
    out = tmp_path / "traffic.md"
    bench.summarize_calls([str(tmp_path / "f"), str(tmp_path / "w")], str(meta), str(out),
                          ["cmd"], WL, algo)
    rows = {}
    for line in open(out):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 6 and cells[3].isdigit():
            rows[cells[0]] = cells
    assert "setup" not in rows                      # set-up kernels are not a call
    # snapkv_select: mean of (100 + 100) and (110 + 90) KiB fetched at scale 2, 2 kernels x 1 KiB written
    assert int(rows["snapkv_select"][1]) == 200 * 1024 * 2
    assert int(rows["snapkv_select"][2]) == 2 * 1024
    assert float(rows["snapkv_select"][5]) == round((400 * 1024 + 2048) / (400 * 1024), 4)
    assert int(rows["verify"][3]) == 404 * 1024 * 2 + 2 * 1024
    assert int(rows["kv_append"][3]) == 3 * 1024 * 2 + 1024     # the index kernel is dropped


def test_call_summary_rejects_a_marker_count_mismatch(tmp_path):
    import pytest
    mark = "kvss::(anonymous namespace)::philox_kernel(x)"
    _marked_run(str(tmp_path / "f"), "FETCH_SIZE", [(mark, 0.0), ("kvss::a(x)", 1.0)])
    with pytest.raises(ValueError):
        bench.split_calls(str(tmp_path / "f"), ["verify", "draft_snapkv"])


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


def test_committed_traffic_is_per_workload_and_source():
    # a workload with no committed counter summary reports no traffic
    assert bench.committed_call_traffic("tiny_fp32") == {}
    assert bench.calls_summary_path("llama8b_ctx32k").endswith(
        os.path.join("profiles", "traffic_llama8b_ctx32k.md"))
