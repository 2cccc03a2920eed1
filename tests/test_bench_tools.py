"""CPU checks of the benchmark's profile tooling: the kernel labels of the
trace summary, its steady-state averages, the calibration of the FETCH_SIZE /
WRITE_SIZE traffic figures, and the source-hash guard that keeps a stale
traffic record out of the benchmark line.  Inputs are small synthetic
rocprofv3 csv files in the columns the profiler writes."""
import csv
import json
import os

import pytest

import bench

TRACE_COLS = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id",
              "Kernel_Id", "Kernel_Name", "Correlation_Id", "Start_Timestamp", "End_Timestamp",
              "LDS_Block_Size", "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count",
              "Workgroup_Size_X", "Workgroup_Size_Y", "Workgroup_Size_Z", "Grid_Size_X",
              "Grid_Size_Y", "Grid_Size_Z"]
PMC_COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
            "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
            "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
            "Counter_Value", "Start_Timestamp", "End_Timestamp"]
FWD = "_ZN3sas10fwd_kernelIDF16bDF16bLi128ELi4ELb0EEEvNS_9FwdParamsE"


def write_csv(path, cols, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow({c: r.get(c, 0) for c in cols})


@pytest.mark.parametrize("name,label", [
    (FWD, "fwd_kernel<bf16, bf16, 128, 4, false>"),
    ("_ZN3sas19select_merge_kernelILi4ELi256EEEvNS_12DecodeParamsENS_12SelectParamsE",
     "select_merge_kernel<4, 256>"),
    ("_ZN3sas14append_kernelEv", "sas::append_kernel"),
    ("sas::bwd_csr_kernel(sas::BwdParams)", "sas::bwd_csr_kernel"),
    ("void (anonymous namespace)::read_chunk_kernel<8>(HIP_vector_type<unsigned int, 4u> "
     "const*, long, unsigned int*)", "peaks::read_chunk_kernel<8>"),
    ("(anonymous namespace)::mfma_loop_kernel(int, float*)", "peaks::mfma_loop_kernel"),
    ("__amd_rocclr_fillBufferAligned", "__amd_rocclr_fillBufferAligned (HIP runtime)"),
    ("void at::native::(anonymous namespace)::distribution_elementwise_grid_stride_kernel<float, "
     "4>(long)", "at::native::(anonymous namespace)::distribution_elementwise_grid_stride_kernel "
     "(torch)"),
])
def test_kernel_labels(name, label):
    assert bench.kernel_label(name) == label


def test_short_kernel_names_only_library_kernels():
    assert bench.short_kernel(FWD) == "fwd_kernel"
    assert bench.short_kernel("sas::bwd_csr_kernel(sas::BwdParams)") == "bwd_csr_kernel"
    assert bench.short_kernel("__amd_rocclr_copyBuffer") == "copyBuffer"
    assert bench.short_kernel("(anonymous namespace)::read_kernel(long)") is None


def test_trace_summary_steady_state(tmp_path):
    """Seven dispatches of one kernel (10, 10, 100, 4, 4, 4, 4 us) with the
    first two left out: the steady average is (100 + 4 * 4) / 5 = 23.2 us;
    another launch grid of the same kernel gets its own row."""
    durs = [10, 10, 100, 4, 4, 4, 4]
    rows, t = [], 1000
    for i, d in enumerate(durs):
        rows.append({"Kind": "KERNEL_DISPATCH", "Dispatch_Id": i + 1, "Kernel_Name": FWD,
                     "Start_Timestamp": t, "End_Timestamp": t + 1000 * d,
                     "Workgroup_Size_X": 512, "Workgroup_Size_Y": 1, "Workgroup_Size_Z": 1,
                     "Grid_Size_X": 512 * 1280, "Grid_Size_Y": 8, "Grid_Size_Z": 1,
                     "LDS_Block_Size": 68096, "VGPR_Count": 108})
        t += 1000 * d + 500
    rows.append({"Kind": "KERNEL_DISPATCH", "Dispatch_Id": 99, "Kernel_Name": FWD,
                 "Start_Timestamp": t, "End_Timestamp": t + 7000, "Workgroup_Size_X": 512,
                 "Workgroup_Size_Y": 1, "Workgroup_Size_Z": 1, "Grid_Size_X": 512 * 256,
                 "Grid_Size_Y": 8, "Grid_Size_Z": 1})
    write_csv(str(tmp_path / "tr" / "run_kernel_trace.csv"), TRACE_COLS, rows)
    out = str(tmp_path / "trace.md")
    bench.summarize_trace(str(tmp_path / "tr"), "cmd", out, skip=2)
    rec = json.load(open(str(tmp_path / "trace.json")))["kernels"]
    big = rec["fwd_kernel<bf16, bf16, 128, 4, false> [10240 WGs]"]
    assert big["calls"] == 7
    assert big["avg_us"] == pytest.approx(sum(durs) / 7)
    assert big["steady_avg_us"] == pytest.approx(23.2)
    small = rec["fwd_kernel<bf16, bf16, 128, 4, false> [2048 WGs]"]
    assert small["calls"] == 1 and small["steady_avg_us"] == pytest.approx(7.0)
    assert "`fwd_kernel<bf16, bf16, 128, 4, false>` | 10240 | 7 |" in open(out).read()


def pmc_rows(counter, copy_kib, kern_kib):
    rows = [{"Dispatch_Id": i, "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": counter,
             "Counter_Value": v} for i, v in enumerate([3.0, 1.5] + [copy_kib] * 3)]
    rows += [{"Dispatch_Id": 10 + i, "Kernel_Name": FWD, "Counter_Name": counter,
              "Counter_Value": v} for i, v in enumerate(kern_kib)]
    return rows


def test_traffic_calibration_and_hash_guard(tmp_path, monkeypatch):
    """The 1 GiB copy reads 524288 KiB by FETCH_SIZE (half the bytes) and
    writes 1048576 KiB: the fetch counter is scaled by 2, the write counter
    by 1, so a kernel reading 1000 (and 1200) KiB and writing 500 KiB moves
    1100 * 1024 * 2 + 500 * 1024 bytes per launch.  The record is tagged with
    the current source hash; any other hash or workload yields no traffic."""
    tj = str(tmp_path / "traffic.json")
    monkeypatch.setattr(bench, "TRAFFIC_JSON", tj)
    write_csv(str(tmp_path / "f" / "run_counter_collection.csv"), PMC_COLS,
              pmc_rows("FETCH_SIZE", 524288.0, [1000.0, 1200.0]))
    write_csv(str(tmp_path / "w" / "run_counter_collection.csv"), PMC_COLS,
              pmc_rows("WRITE_SIZE", 1048576.0, [500.0, 500.0]))
    bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), "cmd",
                        str(tmp_path / "traffic.md"), "varlen")
    rec = json.load(open(tj))
    assert rec["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert rec["calibration"]["write_factor"] == pytest.approx(1.0)
    want = 1100 * 1024 * 2 + 500 * 1024
    assert rec["kernels"]["fwd_kernel"]["bytes_per_launch"] == want
    assert rec["source_hash"] == bench.source_hash()
    assert bench.traffic_for("fwd_kernel", "varlen") == want
    assert bench.traffic_for("fwd_kernel", "layer16k") is None
    assert bench.traffic_for("bwd_dq_kernel", "varlen") is None
    rec["source_hash"] = "0" * 16
    json.dump(rec, open(tj, "w"))
    assert bench.traffic_for("fwd_kernel", "varlen") is None


def test_source_hash_ignores_comments_only():
    c = "int f(int x) {\n  // the answer\n  return x + 1; /* done */\n}\n"
    assert bench._code_only(c) == bench._code_only("int f(int x){return x+1;}")
    assert bench._code_only(c) != bench._code_only("int f(int x){return x+2;}")
    assert bench._code_only("x = 1  # one\n# note\n", python=True) == \
        bench._code_only("x = 1  # one\n", python=True)


def test_more_than_one_gpu_is_refused_with_a_message():
    """The benchmark measures one GPU: --gpus above 1 exits non-zero, before
    touching any device, and says why."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
