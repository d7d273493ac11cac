"""CPU tests of bench.py's host logic: the one-GPU guard and the profile
summarisers (kernel series of the configuration sweep, a K-split GEMM's
partial-sum kernel counted with its launch, shader-counter derivations),
run on small synthetic rocprofv3 CSV files."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2 and "single MI355X" in r.stderr and "--gpus 2" in r.stderr


def write_trace(path, launches):
    """launches: (kernel name, duration us), back to back."""
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "1_kernel_trace.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        t = 1000
        for name, us in launches:
            w.writerow([f"void {name}(K2Args)", t, t + int(us * 1000)])
            t += int(us * 1000) + 500


def test_config_summary_series_and_k_split(tmp_path):
    per = 8 + 50 + 5 * 24
    launches = [("k1_quantize_lowrank_down<1, false>", 10.0)] * per
    launches += [("k2_w4a4_gemm<0, 0, false, false, false, false>", 100.0)] * per
    launches += [("k1_quantize_lowrank_down<4, false>", 11.0)] * per
    for _ in range(per):                         # K-split GEMM: two kernels per launch
        launches += [("k2_w4a4_gemm<0, 0, true, false, false, true>", 30.0), ("k2_split_sum<0, false>", 15.0)]
    write_trace(str(tmp_path / "trace"), launches)
    cfg = tmp_path / "cfg.jsonl"
    cfg.write_text("\n".join(json.dumps(d) for d in [
        {"config": "big", "M": 4608, "N": 3072, "K": 3072, "rank": 32},
        {"config": "small", "M": 1024, "N": 3072, "K": 3072, "rank": 128}]) + "\n")
    out = tmp_path / "summary.md"
    bench.summarize_configs(str(tmp_path / "trace"), str(cfg), str(out), "cmd")
    rows = [l for l in out.read_text().splitlines() if l.startswith("| big") or l.startswith("| small")]
    assert len(rows) == 4
    cells = [[c.strip() for c in r.split("|")] for r in rows]
    assert cells[1][3] == "100.00"                # big K2
    assert cells[3][3] == "45.00"                 # small K2: GEMM + partial sum, one launch
    tops = 2.0 * 1024 * 3072 * 3072 / 45.0 / 1e6
    assert cells[3][6] == f"{tops:.0f} TOPS"


def test_counter_summary(tmp_path):
    d = tmp_path / "pmc" / "x"
    d.mkdir(parents=True)
    vals = {"GRBM_GUI_ACTIVE": 8 * 1000.0, "SQ_WAVES": 64, "SQ_BUSY_CYCLES": 1, "SQ_INSTS_VALU": 1024 * 100 + 50,
            "SQ_INSTS_MFMA": 50, "SQ_VALU_MFMA_BUSY_CYCLES": 1024 * 250.0, "SQ_ACTIVE_INST_VALU": 1}
    with open(d / "1_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
                    "End_Timestamp"])
        for disp in (1, 2):
            for c, v in vals.items():
                w.writerow([disp, "void k2_w4a4_gemm<0, 1, false, false, true, false>(K2Args)", c, v, 0, 5000])
    out = tmp_path / "c.md"
    bench.summarize_counters(str(tmp_path / "pmc"), str(out), "cmd")
    row = [l for l in out.read_text().splitlines() if l.startswith("| `k2")][0]
    cells = [c.strip() for c in row.split("|")]
    assert cells[2] == "2" and cells[3] == "5.0" and cells[4] == "1000"
    assert cells[-3] == "40%"                    # 1024 * 100 vector instructions x 4 / (1024 x 1000)
    assert cells[-2] == "25%"                    # 1024 * 250 matrix cycles / (1024 x 1000)
