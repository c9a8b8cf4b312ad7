"""The rocprofv3 summary tool on small hand-made CSV files: per-dispatch sums over
counter instances, the copy-calibrated traffic figure that bench.py reports as
roofline.traffic, and the ratios of the counter summaries."""
import argparse
import csv

import pytest

import bench_profile


COUNTER_FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id",
                  "Thread_Id", "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size",
                  "LDS_Block_Size", "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count",
                  "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp",
                  "End_Timestamp"]


def write_counters(path, rows):
    """rows: (dispatch, kernel, counter, value, start_ns, end_ns)"""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COUNTER_FIELDS)
        w.writeheader()
        for d, k, c, v, t0, t1 in rows:
            w.writerow({"Correlation_Id": d, "Dispatch_Id": d, "Agent_Id": "Agent 1", "Queue_Id": 1,
                        "Process_Id": 1, "Thread_Id": 1, "Grid_Size": 65536, "Kernel_Id": 1,
                        "Kernel_Name": k, "Workgroup_Size": 256, "LDS_Block_Size": 0,
                        "Scratch_Size": 0, "VGPR_Count": 0, "Accum_VGPR_Count": 0,
                        "SGPR_Count": 0, "Counter_Name": c, "Counter_Value": v,
                        "Start_Timestamp": t0, "End_Timestamp": t1})


def test_per_dispatch_sums_instances_and_filters_kernels(tmp_path):
    p = tmp_path / "c.csv"
    write_counters(p, [
        (1, "void gemm_a(x)", "FETCH_SIZE", 10.0, 0, 1000),
        (1, "void gemm_a(x)", "FETCH_SIZE", 5.0, 0, 1000),   # a second instance (another XCD)
        (2, "void other(x)", "FETCH_SIZE", 99.0, 0, 1000),
        (3, "void gemm_a(x)", "FETCH_SIZE", 7.0, 0, 1000),
        (3, "void gemm_a(x)", "WRITE_SIZE", 1.0, 0, 1000),
    ])
    assert bench_profile.per_dispatch(str(p), "FETCH_SIZE", "gemm_a") == [15.0, 7.0]
    assert bench_profile.per_dispatch(str(p), "WRITE_SIZE", "gemm_a") == [1.0]
    assert bench_profile.per_dispatch(str(p), "FETCH_SIZE", "nothing") == []


def test_traffic_is_calibrated_by_the_copy(tmp_path):
    """A copy of N bytes whose counters read N/2 (fetch) and N (write) KiB-units gives
    factors 2 and 1; the GEMM's medians (first two dispatches skipped) are scaled by them."""
    gf, gw, cf, cw = (tmp_path / n for n in ("gf.csv", "gw.csv", "cf.csv", "cw.csv"))
    k = "tile16_gemm<dmp::BF16, true, true>"
    write_counters(gf, [(d, k, "FETCH_SIZE", v, 0, 1) for d, v in
                        enumerate([1.0, 2.0, 100.0, 101.0, 99.0], 1)])
    write_counters(gw, [(d, k, "WRITE_SIZE", v, 0, 1) for d, v in
                        enumerate([3.0, 4.0, 50.0, 50.0, 50.0], 1)])
    nbytes = 1024.0 * 1024
    write_counters(cf, [(d, "copyBuffer", "FETCH_SIZE", nbytes / 2 / 1024, 0, 1) for d in (1, 2, 3)])
    write_counters(cw, [(d, "copyBuffer", "WRITE_SIZE", nbytes / 1024, 0, 1) for d in (1, 2, 3)])
    out = tmp_path / "t.md"
    a = argparse.Namespace(gemm_fetch=str(gf), gemm_write=str(gw), copy_fetch=str(cf),
                           copy_write=str(cw), copy_bytes=nbytes, kernel=k,
                           copy_kernel="copyBuffer", cmd="test", out=str(out))
    bench_profile.cmd_traffic(a)
    text = out.read_text()
    assert "calibration factors (known bytes / counter bytes): fetch 2.0000, write 1.0000" in text
    total, digest = bench_profile.read_traffic(str(out))
    # fetch median of (100, 101, 99) KiB x 2, write 50 KiB x 1
    assert total == pytest.approx(100 * 1024 * 2 + 50 * 1024, abs=1)
    assert digest == bench_profile.kernel_source_hash()


def test_counter_ratios(tmp_path):
    """MFMA busy = busy cycles / (1024 SIMDs x cycles per XCD); clock = cycles per XCD /
    launch time; bank conflicts relative to LDS-active cycles."""
    p = tmp_path / "k.csv"
    k = "tile16_gemm<dmp::I8"
    cyc_per_xcd = 200000.0
    rows = []
    for d in range(1, 6):
        rows += [(d, k, "GRBM_GUI_ACTIVE", 8 * cyc_per_xcd, 0, 100_000),   # 100 us
                 (d, k, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * 1024 * cyc_per_xcd, 0, 100_000),
                 (d, k, "SQ_LDS_IDX_ACTIVE", 1000.0, 0, 100_000),
                 (d, k, "SQ_LDS_BANK_CONFLICT", 250.0, 0, 100_000),
                 (d, k, "TCC_HIT_sum", 3.0, 0, 100_000),
                 (d, k, "TCC_MISS_sum", 1.0, 0, 100_000)]
    write_counters(p, rows)
    out = tmp_path / "k.md"
    a = argparse.Namespace(csv=[str(p)], kernel=k, cmd="test", out=str(out), us=None)
    bench_profile.cmd_counters(a)
    text = out.read_text()
    assert "cycles per XCD (GRBM_GUI_ACTIVE / 8): 200000" in text
    assert "effective clock 2.00 GHz" in text
    assert "MFMA busy (per SIMD): 50.0 %" in text
    assert "(SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE): 25.00 %" in text
    assert "L2 hit rate: 75.0 %" in text
    assert f"kernel_source_sha256: {bench_profile.kernel_source_hash()}" in text


def test_stats_table(tmp_path):
    p = tmp_path / "s.csv"
    with open(p, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs",
                    "StdDev"])
        w.writerow(["void dmp::tile16_gemm<dmp::BF16, true, true>(dmp::TileArgs)", 10, 1070000,
                    107000.0, 99.0, 105000, 120000, 1.0])
    out = tmp_path / "s.txt"
    bench_profile.cmd_stats(argparse.Namespace(csv=str(p), cmd="the command", out=str(out)))
    text = out.read_text()
    assert "command: the command" in text
    line = [x for x in text.splitlines() if x.startswith("void dmp::tile16_gemm")][0]
    assert line.split()[-5:] == ["10", "107.00", "105.00", "120.00", "99.00"]

