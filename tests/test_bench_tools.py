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
    all_rows = [l for l in out.read_text().splitlines() if l.startswith("| big") or l.startswith("| small")]
    rows = [l for l in all_rows if "layer (K1 + K2)" not in l]
    layers = [[c.strip() for c in l.split("|")] for l in all_rows if "layer (K1 + K2)" in l]
    assert len(rows) == 4 and len(layers) == 2
    assert layers[0][3] == "110.00"               # big: 10 + 100 us
    assert layers[1][3] == "56.00"                # small: 11 + 45 us
    cells = [[c.strip() for c in r.split("|")] for r in rows]
    assert cells[1][3] == "100.00"                # big K2
    assert cells[3][3] == "45.00"                 # small K2: GEMM + partial sum, one launch
    tops = 2.0 * 1024 * 3072 * 3072 / 45.0 / 1e6
    assert cells[3][6] == f"{tops:.0f} TOPS ({tops / bench.PEAK_INT8_TOPS:.1%} of int8)"
    assert cells[3][7] == f"{tops / bench.PEAK_FP6_TOPS:.1%}"     # INT4 codes run as fp6


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


def test_counter_summary_of_waits_and_lds(tmp_path):
    d = tmp_path / "pmc" / "x"
    d.mkdir(parents=True)
    vals = {"GRBM_GUI_ACTIVE": 8 * 1000.0, "SQ_WAVE_CYCLES": 4000.0, "SQ_WAIT_ANY": 1000.0,
            "SQ_WAIT_INST_ANY": 2000.0, "SQ_ACTIVE_INST_ANY": 800.0, "SQ_INSTS_LDS": 500.0,
            "SQ_WAIT_INST_LDS": 40.0, "SQ_LDS_BANK_CONFLICT": 25.0}
    with open(d / "1_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
                    "End_Timestamp"])
        for c, v in vals.items():
            w.writerow([1, "void k2_w4a4_gemm<0, 0, false, true, false, false>(K2Args)", c, v, 0, 3000])
            w.writerow([1, "void some_other_kernel(int)", c, v, 0, 3000])
    out = tmp_path / "m.md"
    bench.summarize_counters_mem(str(tmp_path / "pmc"), str(out), "cmd")
    rows = [l for l in out.read_text().splitlines() if l.startswith("| `")]
    assert len(rows) == 1                        # the library's kernels only
    cells = [c.strip() for c in rows[0].split("|")]
    assert cells[3] == "3.0" and cells[4] == "1000"
    assert cells[-6:-1] == ["25%", "50%", "20%", "1.0%", "0.050"]


def test_mfma_summary(tmp_path):
    j = tmp_path / "m.jsonl"
    j.write_text(json.dumps({"mfma": "fp6 32x32x64", "grid": 512, "iters": 10, "ms": 7.0, "rate_tops": 9065.8,
                             "peak_tops": 10100.0, "frac_of_peak": 0.8976, "sclk_mhz": None,
                             "ns_per_instruction_per_simd": 14.1}) + "\n")
    out = tmp_path / "p.md"
    bench.summarize_mfma(str(j), str(out), "cmd")
    row = [l for l in out.read_text().splitlines() if l.startswith("| fp6")][0]
    assert [c.strip() for c in row.split("|")][2:6] == ["7.000", "9066", "10100", "89.8%"]
    # with the instruction mixes: the overlap ratio and the GEMM step's floor
    with open(j, "a") as f:
        f.write("\n" + json.dumps({"mix": "a", "kind": 5, "grid": 512, "iters": 10, "ms": 1.0,
                                    "ns_per_slot_per_simd": 30.0}))
        f.write("\n" + json.dumps({"mix": "b", "kind": 6, "grid": 512, "iters": 10, "ms": 1.0,
                                    "ns_per_slot_per_simd": 20.0}))
        f.write("\n" + json.dumps({"mix": "c", "kind": 7, "grid": 512, "iters": 10, "ms": 1.0,
                                    "ns_per_slot_per_simd": 50.0}))
    bench.summarize_mfma(str(j), str(out), "cmd")
    text = out.read_text()
    assert "together, on independent registers, 30.00 ns, 88% of their sum" in text   # 30 / (14.1 + 20)
    assert "three parts" not in text              # no bf16 32x32x8 row yet
    with open(j, "a") as f:
        f.write("\n" + json.dumps({"mfma": "bf16 32x32x8", "grid": 512, "iters": 10, "ms": 1.0, "rate_tops": 1.0,
                                    "peak_tops": 2500.0, "frac_of_peak": 0.5, "ns_per_instruction_per_simd": 10.9}))
    bench.summarize_mfma(str(j), str(out), "cmd")
    assert "takes 50.00 ns against 45.00 ns for its three parts alone (111%)" in out.read_text()
    assert "a wavefront's group (8 tiles) 400 ns" in text and "that is 154 us" in text


def test_summaries_refuse_mixed_runs(tmp_path):
    """A profile directory holding two runs' CSV files is refused rather than
    summarised from whichever file the walk meets first."""
    d = tmp_path / "trace" / "vm"
    write_trace(str(d), [("k2_w4a4_gemm<0>", 10.0)])
    assert bench._find(str(tmp_path / "trace"), "kernel_trace.csv").endswith("1_kernel_trace.csv")
    with open(d / "2_kernel_trace.csv", "w") as f:
        f.write("Kernel_Name,Start_Timestamp,End_Timestamp\n")
    with pytest.raises(RuntimeError, match="several runs"):
        bench._find(str(tmp_path / "trace"), "kernel_trace.csv")
    with pytest.raises(FileNotFoundError):
        bench._find(str(tmp_path / "trace"), "kernel_stats.csv")


def test_gemm_mix_ceiling():
    """The busiest CU's share of the GEMM: fc1 (4608 x 12288, K = 3072) has
    1728 tiles, 7 on the busiest CU, 48 groups each; fc2 (4608 x 3072, K =
    12288) 432 tiles, 2 on the busiest CU, 192 groups; 8 steps per group."""
    assert bench.k2_mix_ceiling_us(40.0, 4608, 12288, 3072) == pytest.approx(7 * 48 * 8 * 40.0 / 1e3)
    assert bench.k2_mix_ceiling_us(40.0, 4608, 3072, 12288) == pytest.approx(2 * 192 * 8 * 40.0 / 1e3)
    assert bench.k2_mix_ceiling_us(40.0, 1, 256, 64) == pytest.approx(8 * 40.0 / 1e3)   # one tile, one group
