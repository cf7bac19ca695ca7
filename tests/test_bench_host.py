"""Host-only checks of bench.py's profile summaries: the counter calibration and the
trace table, on small synthetic rocprofv3 CSV files (no GPU)."""

import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _write(path, fields, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _bench(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, check=True)
    return r.stdout


def test_traffic_summary_calibrates_on_the_copy(tmp_path):
    # the 1 GiB copy reads FETCH_SIZE = 524288 (KiB units of 2 KiB) and WRITE_SIZE = 1048576
    f = ["Kernel_Name", "Counter_Value"]
    fetch = [{"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Value": 524288},
             {"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Value": 4},
             {"Kernel_Name": "void moe::k_a<1>(int)", "Counter_Value": 1000},
             {"Kernel_Name": "void moe::k_a<1>(int)", "Counter_Value": 3000},
             {"Kernel_Name": "void other(int)", "Counter_Value": 77}]
    write = [{"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Value": 1048576},
             {"Kernel_Name": "void moe::k_a<1>(int)", "Counter_Value": 500}]
    _write(tmp_path / "f.csv", f, fetch)
    _write(tmp_path / "w.csv", f, write)
    out = _bench("--summarize-traffic", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    assert "FETCH_SIZE x 2.000 KiB and WRITE_SIZE x 1.000 KiB" in out
    # mean fetch 2000 units x 2 KiB = 4,096,000 bytes; write 500 KiB = 512,000 bytes
    assert "| `moe::k_a<1>` | 2 | 4.1 | 0.5 |" in out
    assert "other" not in out


def test_mfma_summary(tmp_path):
    f = ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Counter_Name",
         "Counter_Value"]
    rows = []
    # 100 us at 2.0 GHz: GRBM_GUI_ACTIVE = 8 XCDs x 200,000 cycles; MFMA busy half the
    # SIMD cycles at that clock; 1e9 MOPS -> 512 GFLOP
    for c, v in (("SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 2.0e9 * 1e-4 / 2), ("SQ_INSTS_VALU_MFMA_MOPS_BF16", 1e9),
                 ("GRBM_GUI_ACTIVE", 8 * 2.0e9 * 1e-4)):
        rows.append({"Dispatch_Id": 1, "Kernel_Name": "void moe::gemm_x<2>(B)", "Start_Timestamp": 0,
                     "End_Timestamp": 100000, "Counter_Name": c, "Counter_Value": v})
    _write(tmp_path / "m.csv", f, rows)
    out = _bench("--summarize-mfma", str(tmp_path / "m.csv"), "--algo", "gemm_x=500.0")
    assert "| `moe::gemm_x<2>` | 1 | 512.0 | 500.0 | 100.0 | 41.7% | 2.00 | 50.0% |" in out


def test_trace_summary(tmp_path):
    f = ["Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    rows = [{"Kernel_Name": "void moe::k<1>(int)", "Start_Timestamp": 0, "End_Timestamp": d}
            for d in (1000, 3000, 5000)]
    _write(tmp_path / "t.csv", f, rows)
    out = _bench("--summarize-trace", str(tmp_path / "t.csv"), "--last", "2")
    assert "| `moe::k<1>` | 3 | 4.0 | 3.0 | 5.0 | 3.0 |" in out
