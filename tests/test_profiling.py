"""Host logic of the rocprofv3 summary helper (synthetic CSV files)."""
import csv
import json
import os

from bit_block_quantized_gguf_amd import profiling

PMC_HDR = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
           "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
           "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
           "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _pmc(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=PMC_HDR)
        w.writeheader()
        for i, (name, grid, counter, value) in enumerate(rows):
            r = {k: 0 for k in PMC_HDR}
            r.update({"Dispatch_Id": i, "Grid_Size": grid, "Kernel_Name": name,
                      "Counter_Name": counter, "Counter_Value": value})
            w.writerow(r)


def test_traffic_scaled_by_calibration(tmp_path):
    fdir, wdir = str(tmp_path / "f"), str(tmp_path / "w")
    _pmc(os.path.join(fdir, "x_counter_collection.csv"), [
        ("k<1>", 100, "FETCH_SIZE", 1000.0), ("k<1>", 100, "FETCH_SIZE", 1200.0),
        ("k<1>", 200, "FETCH_SIZE", 9999.0),                       # other shape: filtered
        ("copyBuffer", 7, "FETCH_SIZE", 512.0)])                   # 1 MiB copy reads as 512 KiB
    _pmc(os.path.join(wdir, "y_counter_collection.csv"), [
        ("k<1>", 100, "WRITE_SIZE", 10.0), ("copyBuffer", 7, "WRITE_SIZE", 1024.0)])
    r = profiling.traffic(fdir, wdir, "k<1>", 100, "copyBuffer", 1 << 20)
    assert r["scale"] == {"fetch": 2.0, "write": 1.0}
    assert r["fetch_bytes_per_launch"] == 1100.0 * 1024 * 2
    assert r["write_bytes_per_launch"] == 10.0 * 1024
    assert r["hbm_bytes_per_launch"] == 1100.0 * 2048 + 10240
    assert r["dispatches"] == {"fetch": 2, "write": 1}


def test_traffic_cli_writes_record(tmp_path):
    fdir, wdir = str(tmp_path / "f"), str(tmp_path / "w")
    _pmc(os.path.join(fdir, "a_counter_collection.csv"), [
        ("k", 5, "FETCH_SIZE", 100.0), ("cp", 1, "FETCH_SIZE", 100.0)])
    _pmc(os.path.join(wdir, "b_counter_collection.csv"), [
        ("k", 5, "WRITE_SIZE", 1.0), ("cp", 1, "WRITE_SIZE", 100.0)])
    out = str(tmp_path / "t.json")
    assert profiling.main(["traffic", "--fetch", fdir, "--write", wdir, "--kernel", "k",
                           "--grid", "5", "--calib-kernel", "cp", "--calib-bytes", "102400",
                           "--algorithmic-bytes", "51200", "--source-hash", "abc",
                           "--out", out]) == 0
    rec = json.load(open(out))
    assert rec["hbm_bytes_per_launch"] == 102400 + 1024
    assert rec["traffic_over_algorithmic"] == (102400 + 1024) / 51200
    assert rec["source_hash"] == "abc"


def test_dispatch_filter(tmp_path):
    d = tmp_path / "t"
    d.mkdir()
    with open(d / "r_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X"])
        w.writerow(["gemv_kernel<1>", 100, 1100, 64])
        w.writerow(["gemv_kernel<1>", 2000, 5000, 64])
        w.writerow(["gemv_kernel<1>", 6000, 6500, 128])
        w.writerow(["other", 0, 10, 64])
    rows = profiling.dispatches(str(d), "gemv_kernel", 64)
    assert [r["ns"] for r in rows] == [1000, 3000]


def test_calls_group_consecutive_dispatches(tmp_path):
    """Dispatches are grouped into calls that start at the `start` kernel and
    take the following `include` kernels; unrelated kernels in between are
    skipped, and calls are keyed by the first grid and the kernel sequence."""
    d = tmp_path / "c"
    d.mkdir()
    with open(d / "r_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size"])
        # shape A, two calls (the second out of time order in the file)
        w.writerow(["void q4k::(anonymous namespace)::to_bf16_kernel(float const*)", 0, 1000, 10])
        w.writerow(["void q4k::(anonymous namespace)::gemm_kernel<4>(x)", 1000, 5000, 7])
        w.writerow(["copy", 5000, 5100, 3])                              # not included
        w.writerow(["void q4k::(anonymous namespace)::gemm_fixup_kernel<4>(x)", 5100, 6100, 7])
        w.writerow(["void q4k::(anonymous namespace)::gemm_kernel<4>(x)", 11000, 17000, 7])
        w.writerow(["void q4k::(anonymous namespace)::to_bf16_kernel(float const*)", 10000, 11000, 10])
        w.writerow(["void q4k::(anonymous namespace)::gemm_fixup_kernel<4>(x)", 17000, 19000, 7])
        # shape B, one call without a fix-up
        w.writerow(["void q4k::(anonymous namespace)::to_bf16_kernel(float const*)", 20000, 22000, 20])
        w.writerow(["void q4k::(anonymous namespace)::gemm_kernel<8>(x)", 22000, 30000, 7])
    res = {g["grid"]: g for g in profiling.calls(str(d), "to_bf16_kernel", "gemm")}
    a, b = res[10], res[20]
    assert a["kernels"] == ["to_bf16_kernel", "gemm_kernel<4>", "gemm_fixup_kernel<4>"]
    assert a["calls"] == 2
    assert a["median_us"] == [1.0, 5.0, 1.5]
    assert a["median_sum_us"] == 7.5
    assert b["kernels"] == ["to_bf16_kernel", "gemm_kernel<8>"] and b["calls"] == 1
    assert b["median_sum_us"] == 10.0


def test_calls_alternative_starts_keyed_by_all_grids(tmp_path):
    """A call may start at any of several kernels ('|'); calls whose first
    kernel has the same grid stay apart when a later kernel's grid differs."""
    d = tmp_path / "c"
    d.mkdir()
    with open(d / "r_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size"])
        # two shapes of 32-token calls (no rounding prologue): same main grid,
        # fix-up grids 68 and 20
        w.writerow(["void q4k::(anonymous namespace)::gemm_kernel<1>(x)", 0, 2000, 65536])
        w.writerow(["void q4k::(anonymous namespace)::gemm_fixup_kernel<1>(x)", 2000, 2500, 68])
        w.writerow(["void q4k::(anonymous namespace)::gemm_kernel<1>(x)", 3000, 5000, 65536])
        w.writerow(["void q4k::(anonymous namespace)::gemm_fixup_kernel<1>(x)", 5000, 5700, 20])
        # a call that does start with the prologue
        w.writerow(["void q4k::(anonymous namespace)::to_bf16_kernel(float const*)", 6000, 7000, 10])
        w.writerow(["void q4k::(anonymous namespace)::gemm_kernel<4>(x)", 7000, 9000, 65536])
    res = {tuple(g["grids"]): g for g in
           profiling.calls(str(d), "to_bf16_kernel|gemm_kernel<1>", "gemm")}
    assert set(res) == {(65536, 68), (65536, 20), (10, 65536)}
    assert res[(65536, 68)]["median_sum_us"] == 2.5
    assert res[(65536, 20)]["median_sum_us"] == 2.7
    assert res[(10, 65536)]["kernels"] == ["to_bf16_kernel", "gemm_kernel<4>"]
