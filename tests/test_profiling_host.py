"""Host checks of the rocprofv3 summary helpers (dense_tiled_matrix_amd/
profiling.py) on small synthetic counter files: dispatches are grouped by
kernel and grid size, since one kernel instantiation can serve several
workloads of a run, and the traffic figure is each counter scaled by what it
reads for a device copy of known size."""
import csv
import json

from dense_tiled_matrix_amd import profiling as P

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
          "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
          "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
          "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _write(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, grid, counter, value) in enumerate(rows):
            w.writerow({"Correlation_Id": i, "Dispatch_Id": i + 1, "Agent_Id": "Agent 1",
                        "Queue_Id": 1, "Process_Id": 1, "Thread_Id": 1, "Grid_Size": grid,
                        "Kernel_Id": 1, "Kernel_Name": name, "Workgroup_Size": 256,
                        "LDS_Block_Size": 0, "Scratch_Size": 0, "VGPR_Count": 0,
                        "Accum_VGPR_Count": 0, "SGPR_Count": 0, "Counter_Name": counter,
                        "Counter_Value": value, "Start_Timestamp": 1000,
                        "End_Timestamp": 2000})


def test_traffic_separates_workloads_by_grid(tmp_path):
    gemm = "void dtm::gemm_kernel<2>(dtm::GemmArgs)"
    copy = "__amd_rocclr_copyBuffer"
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    # a 512 MiB copy reads FETCH_SIZE 262144 KiB (scale 2) and WRITE_SIZE
    # 524288 KiB (scale 1); a smaller copy in the same run is left out
    _write(fetch, [(copy, 1, "FETCH_SIZE", 262144.0), (copy, 1, "FETCH_SIZE", 1000.0),
                   (gemm, 262144, "FETCH_SIZE", 800.0), (gemm, 262144, "FETCH_SIZE", 1000.0),
                   (gemm, 65536, "FETCH_SIZE", 100.0)])
    _write(write, [(copy, 1, "WRITE_SIZE", 524288.0),
                   (gemm, 262144, "WRITE_SIZE", 128.0), (gemm, 65536, "WRITE_SIZE", 32.0)])
    spec = [P._spec("big=gemm_kernel<2>@262144"), P._spec("small=gemm_kernel<2>@65536"),
            P._spec("all=gemm_kernel<2>")]
    assert spec[0] == ("big", "gemm_kernel<2>", 262144) and spec[2][2] is None
    rec = P.traffic(str(fetch), str(write), 512.0, spec, "h")
    json.dumps(rec)
    assert rec["calibration"]["fetch_scale"] == 2.0 and rec["calibration"]["write_scale"] == 1.0
    big, small, both = (rec["workloads"][k] for k in ("big", "small", "all"))
    assert big["fetch_size_kib"] == 900.0 and big["write_size_kib"] == 128.0
    assert big["hbm_bytes_per_launch"] == (900 * 2 + 128) * 1024
    assert small["hbm_bytes_per_launch"] == (100 * 2 + 32) * 1024
    # without a grid the two workloads' dispatches are averaged together
    assert both["fetch_size_kib"] == (800 + 1000 + 100) / 3


def test_pmc_summary_groups_by_grid(tmp_path):
    k = "void dtm::gemm_kernel<2>(dtm::GemmArgs)"
    path = tmp_path / "busy.csv"
    # GRBM_GUI_ACTIVE summed over 8 XCDs: 8 * 1000 cycles over 1000 ns -> 1 GHz;
    # MFMA busy = busy cycles / (1000 cycles * 1024 SIMDs)
    _write(path, [(k, 262144, "GRBM_GUI_ACTIVE", 8000.0),
                  (k, 262144, "SQ_VALU_MFMA_BUSY_CYCLES", 512000.0),
                  (k, 65536, "GRBM_GUI_ACTIVE", 8000.0),
                  (k, 65536, "SQ_VALU_MFMA_BUSY_CYCLES", 256000.0)])
    # each row is its own dispatch here; group them into two dispatches
    rows = list(csv.DictReader(open(path)))
    for r in rows:
        r["Dispatch_Id"] = "1" if r["Grid_Size"] == "262144" else "2"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        w.writerows(rows)
    text = P.pmc([str(path)])
    assert "grid 262144 threads (1 dispatch records)" in text
    assert "grid 65536 threads (1 dispatch records)" in text
    assert "1.000 GHz" in text
    assert "MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x 1024 SIMDs)): 50.0%" in text
    assert "): 25.0%" in text
