"""Host-side helpers of bench.py (no GPU): the rocprofv3 CSV summaries with
their dispatch windows, and the FETCH/WRITE ingestion with its copy
calibration, on small hand-made CSV files."""
import contextlib
import csv
import io
import os

import bench

TRACE_FIELDS = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id", "Kernel_Id", "Kernel_Name",
                "Correlation_Id", "Start_Timestamp", "End_Timestamp", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
                "Accum_VGPR_Count", "SGPR_Count", "Workgroup_Size_X", "Workgroup_Size_Y", "Workgroup_Size_Z",
                "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
PMC_FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
              "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
              "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _trace(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=TRACE_FIELDS)
        w.writeheader()
        for i, (name, start_ns, dur_ns, gx, gy, wg) in enumerate(rows):
            w.writerow({"Kind": "KERNEL_DISPATCH", "Dispatch_Id": i + 1, "Kernel_Name": name,
                        "Start_Timestamp": start_ns, "End_Timestamp": start_ns + dur_ns, "LDS_Block_Size": 0,
                        "VGPR_Count": 8, "Workgroup_Size_X": wg, "Workgroup_Size_Y": 1, "Workgroup_Size_Z": 1,
                        "Grid_Size_X": gx, "Grid_Size_Y": gy, "Grid_Size_Z": 1})


def _summary(fn, *args):
    out = io.StringIO()
    with contextlib.redirect_stdout(out):
        fn(*args)
    return out.getvalue().splitlines()


def test_trace_summary_grids_names_and_windows(tmp_path):
    p = str(tmp_path / "t.csv")
    _trace(p, [
        ("void tl::w4_gemm_kernel<2, 2, false, 2>(unsigned char const*)", 1000, 2000, 352 * 256, 1, 256),
        ("(anonymous namespace)::empty_kernel()", 4000, 1000, 64, 1, 64),
        ("void tl::attn_decode_kernel<128, false, 4>(float const*)", 6000, 4000, 3 * 256, 16, 256),
        ("void tl::w4_gemm_kernel<2, 2, false, 2>(unsigned char const*)", 11000, 4000, 352 * 256, 1, 256),
    ])
    lines = _summary(bench.summarize_trace, p)
    body = {l.split()[-1] if "empty" in l else " ".join(l.split()[9:]): l.split() for l in lines[1:]}
    gemm = body["void tl::w4_gemm_kernel<2, 2, false, 2>"]
    assert gemm[0] == "2" and float(gemm[1]) == 3.0 and gemm[5] == "352"   # 2 calls, mean 3 us, 352 blocks
    assert body["void tl::attn_decode_kernel<128, false, 4>"][5] == "48"    # 3 x 16 blocks from X*Y
    assert "empty_kernel" in body                                           # anonymous namespace stripped
    until = _summary(bench.summarize_trace, p, "attn_decode_kernel", None)
    assert len(until) == 3 and until[1].split()[0] == "1"                   # first GEMM and the empty kernel
    since = _summary(bench.summarize_trace, p, None, "attn_decode_kernel")
    assert len(since) == 3


def _pmc(dirpath, rows):
    os.makedirs(dirpath, exist_ok=True)
    with open(os.path.join(dirpath, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=PMC_FIELDS)
        w.writeheader()
        for disp, name, grid, counter, value in rows:
            w.writerow({"Dispatch_Id": disp, "Kernel_Name": name, "Grid_Size": grid, "Counter_Name": counter,
                        "Counter_Value": value})


def test_ingest_scales_by_the_copy_and_averages_dispatches(tmp_path):
    gemv = "void tl::w4_gemv_kernel<2, 1, 1, 2, 1, false>(unsigned char const*)"
    copy = "__amd_rocclr_copyBuffer"
    # FETCH reads half the copied bytes (factor 2), WRITE all of them (factor 1)
    _pmc(str(tmp_path / "f"), [(1, gemv, 180224, "FETCH_SIZE", 5000.0), (2, gemv, 180224, "FETCH_SIZE", 7000.0),
                               (3, copy, 131072, "FETCH_SIZE", 131072.0)])
    _pmc(str(tmp_path / "w"), [(1, gemv, 180224, "WRITE_SIZE", 10.0), (2, gemv, 180224, "WRITE_SIZE", 14.0),
                               (3, copy, 131072, "WRITE_SIZE", 262144.0)])
    data = bench._ingest_runs(str(tmp_path / "f"), str(tmp_path / "w"), 256 * 2**20, bench._forward_kernels())
    ent = data["gemv_gate_up"]
    assert ent["fetch_bytes_per_launch"] == 6000 * 1024 * 2
    assert ent["write_bytes_per_launch"] == 12 * 1024
    assert ent["bytes_per_launch"] == 6000 * 1024 * 2 + 12 * 1024
    assert ent["dispatches"] == [2, 2]
    assert "gemm_gate_up" not in data                                        # no such dispatch in these runs


def test_pmc_summary_windows_by_dispatch(tmp_path):
    a = "void tl::w4_gemm_kernel<8, 2, false, 0>(x)"
    b = "void tl::w4_gemv_kernel<1, 0, 1, 2, 1, false>(x)"
    _pmc(str(tmp_path / "k"), [(1, b, 65536, "FETCH_SIZE", 100.0), (2, a, 180224, "FETCH_SIZE", 900.0),
                               (3, b, 65536, "FETCH_SIZE", 300.0)])
    before = _summary(bench.summarize_pmc, [str(tmp_path / "k")], "w4_gemm_kernel<8", None)
    after = _summary(bench.summarize_pmc, [str(tmp_path / "k")], None, "w4_gemm_kernel<8")
    assert len(before) == 2 and float(before[1].split()[-1]) == 100.0
    vals = {l.split("(")[0].strip()[:30]: float(l.split()[-1]) for l in after[1:]}
    assert sorted(vals.values()) == [300.0, 900.0]


def test_gemv_a16_template_follows_the_library_dispatch():
    """The counter ingest finds the M = 1 fp16-input GEMV by template: 2, 6 or 8 groups per wave
    for up to 16, 48 or 64 K groups, fp16 chunks per thread rounded up to a power of 2."""
    t = bench._gemv_a16_template
    assert t(2048) == "w4_gemv_kernel<1, 0, 1, 2, 1, false>"    # QKV / O / gate-up shapes
    assert t(5632) == "w4_gemv_kernel<1, 0, 1, 6, 2, false>"    # down projection, 44 groups
    assert t(6144) == "w4_gemv_kernel<1, 0, 1, 6, 2, false>"    # 48 groups: the last with 6
    assert t(6272) == "w4_gemv_kernel<1, 0, 1, 8, 2, false>"    # 49 groups
    assert t(704) == "w4_gemv_kernel<1, 0, 1, 2, 1, false>"     # tiny shape's down projection


def test_more_than_one_gpu_is_refused_with_a_message():
    """bench.py measures one GPU; asked for more it says so and exits 2
    before touching a device (this host has none)."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""
