"""Host-side logic of bench.py that needs no GPU: the one-GPU guard and the reductions of
rocprofv3 output (cold-call trace, counter runs) on small synthetic files."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

COLD_MD = """# Cold per-call times of the step's HBM-bound calls

Command (run from the repository root on one MI355X):

```
python3 bench.py --cold-md out.md
```

| family | call | MB | per step | µs | GB/s | % of 8 TB/s |
|---|---|---|---|---|---|---|
| slice | qkv P2 | 200.0 | 2 | 40.0 | 5000 | 62.5 |
| sum | P2 f32 | 300.0 | 1 | 60.0 | 5000 | 62.5 |
| gemv | adaLN B1 | 100.0 | 0 | 25.0 | 4000 | 50.0 |

| family (weighted) | GB/s | % of 8 TB/s |
|---|---|---|
| slice | 5000 | 62.5 |
| sum | 5000 | 62.5 |
"""


def _trace(path, rows):
    """rows: (kernel name, duration ns), one after another."""
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        t = 1000
        for name, ns in rows:
            w.writerow([name, t, t + ns])
            t += ns + 500


def test_gpus_above_one_exits_with_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cold_trace_takes_the_dispatches_after_each_flush(tmp_path, capsys):
    md = tmp_path / "cold.md"
    md.write_text(COLD_MD)
    red = "void at::native::reduce_kernel<512, 1>(...)"
    rows = [("copy_segments_kernel<16>", 9000), (red, 100000), ("copy_segments_kernel<16>", 7000)]
    for name, us in (("copy_segments_kernel<16>", [31, 30, 29, 35, 30]),
                     ("combine_sum_kernel<2, false, false>", [50, 51, 49, 52, 50]),
                     ("gemv_bf16_kernel<12, 1>", [20, 19, 21, 20, 20])):
        for u in us:
            rows += [(red, 100000), (name, u * 1000)]
    rows.append(("gemv_bf16_kernel<12, 1>", 15000))   # a warm call after the section
    _trace(tmp_path / "trace.csv", rows)
    bench.cold_trace(str(tmp_path / "trace.csv"), str(md))
    out = capsys.readouterr().out
    # medians 30, 50 and 20 us; 200 MB in 30 us = 6667 GB/s
    assert "| slice | qkv P2 | 200.0 | 2 | 40.0 | 62.5 | 30.0 | 6667 | 83.3 |" in out
    assert "| sum | P2 f32 | 300.0 | 1 | 60.0 | 62.5 | 50.0 | 6000 | 75.0 |" in out
    assert "| gemv | adaLN B1 | 100.0 | 0 | 25.0 | 50.0 | 20.0 | 5000 | 62.5 |" in out
    # weighted over the step (the GEMV row has weight 0): slice only, then sum only
    assert "| slice | 6667 | 83.3 |" in out and "| sum | 6000 | 75.0 |" in out
    assert "| gemv | 5000" not in out


def test_cold_trace_rejects_a_family_mismatch(tmp_path):
    md = tmp_path / "cold.md"
    md.write_text(COLD_MD)
    red = "reduce_kernel"
    rows = []
    for name in ("copy_segments_kernel", "gemv_bf16_kernel", "gemv_bf16_kernel"):   # sum row gets a GEMV
        for _ in range(bench.COLD_REPS):
            rows += [(red, 1000), (name, 1000)]
    _trace(tmp_path / "trace.csv", rows)
    with pytest.raises(SystemExit, match="sum P2 f32"):
        bench.cold_trace(str(tmp_path / "trace.csv"), str(md))


def test_counters_scale_bytes_by_the_calibration_copy(tmp_path, monkeypatch):
    """Two launches (a GEMM and a slice) and the calibration copy; FETCH_SIZE reads half of
    the true bytes on the copy, so every fetch figure is doubled (slice: 512 B counted -> 1024,
    plus 1024 written, over 2000 algorithmic)."""
    cal = 1 << 27
    probe = {"launches": [["gemm", "colwise 8x8x8", 1024.0, 1000.0], ["slice", "w1 P2", 0.0, 2000.0]],
             "cal_bytes": cal}
    pj = tmp_path / "probe.json"
    pj.write_text(json.dumps(probe))
    names = ["gemm4_bf16_nt_kernel<7, 8, true, false, 0>", "copy_segments_kernel<16>", "copy_segments_kernel<16>"]
    runs = {"fetch": ("FETCH_SIZE", [1.0, 0.5, cal / 2048]), "write": ("WRITE_SIZE", [0.5, 1.0, cal / 1024])}
    for tag, (counter, kib) in runs.items():
        d = tmp_path / tag
        d.mkdir()
        with open(d / "run_counter_collection.csv", "w", newline="") as f:
            w = csv.writer(f)
            w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
            w.writerow([1, "at::native::fill", counter, 7.0])          # not a library kernel
            for i, (n, v) in enumerate(zip(names, kib)):
                w.writerow([i + 2, n, counter, v])
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    bench.reduce_counters(str(pj), [str(tmp_path / "fetch"), str(tmp_path / "write")])
    t = json.load(open(tmp_path / "traffic.json"))
    assert t["factors"]["FETCH_SIZE"] == pytest.approx(2.0)
    assert t["factors"]["WRITE_SIZE"] == pytest.approx(1.0)
    assert t["fetch_bytes_per_launch"] == 2048       # 1 KiB counted, factor 2
    assert t["write_bytes_per_launch"] == 512
    assert t["ratio_to_algorithmic"] == pytest.approx(2.56)
    md = open(tmp_path / "profiles" / "dit_block_step_counters.md").read()
    assert "| slice: w1 P2 | 1 | 0.0 | 0.0 | 0.0 | 1.024 |" in md


def test_counters_normalise_issue_counters_per_cu_and_per_wave_cycle(tmp_path, monkeypatch):
    """The issue back-pressure run: a TA FIFO-full count is divided by the CU cycles (GUI-active
    cycles per XCD x 256 CUs: 8000 / 8 x 256), an LDS issue wait by the wave cycles."""
    probe = {"launches": [["gemm", "colwise 8x8x8", 1024.0, 1000.0]], "cal_bytes": 1 << 27}
    pj = tmp_path / "probe.json"
    pj.write_text(json.dumps(probe))
    d = tmp_path / "issue"
    d.mkdir()
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        gemm = "gemm4_bf16_nt_kernel<7, 8, true, false, 0>"
        for c, v in (("GRBM_GUI_ACTIVE", 8000.0), ("SQ_VMEM_TA_ADDR_FIFO_FULL", 25600.0),
                     ("SQ_WAVE_CYCLES", 4000.0), ("SQ_WAIT_INST_LDS", 200.0)):
            w.writerow([1, gemm, c, v])
        w.writerow([2, "copy_segments_kernel<16>", "GRBM_GUI_ACTIVE", 10.0])
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    bench.reduce_counters(str(pj), [str(d)])
    md = open(tmp_path / "profiles" / "dit_block_step_counters.md").read()
    assert "| family: shape | VMEM_TA_ADDR_FIFO_FULL | WAIT_INST_LDS |" in md
    assert "| gemm: colwise 8x8x8 | 0.100 | 0.050 |" in md
    assert bench.ATTR_ISSUE.split()[0] == "SQ_VMEM_TA_ADDR_FIFO_FULL"   # names the run's folder
    assert "pmc_sq_vmem_ta_addr_fifo_full" in md


def _pmc_run(path, rows):
    """rows: (dispatch id, kernel name, counter, value, duration ns)."""
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value",
                    "Start_Timestamp", "End_Timestamp"])
        for disp, name, counter, value, ns in rows:
            w.writerow([disp, 1024, name, counter, value, 1000, 1000 + ns])


def test_pmc_summary_labels_dispatches_by_their_flops(tmp_path, capsys):
    """Two runs of one program: the flops counted in the first label the same dispatch ids in
    the second, so two shapes of one kernel and grid get separate rows; hipBLASLt kernels get a
    short label and other kernels are left out."""
    ours = "void tpl::(anonymous namespace)::gemm4_bf16_nt_kernel<8, 8, true, false, 0>(tpl::GemmParams)"
    vend = "Cijk_Alik_Bljk_BBS_BH_Bias_HA_S_SAV_UserArgs_MT256x256x64_MI16x16x1_SK3_gfx950"
    other = "void at::native::elementwise_kernel<128, 4>(...)"
    _pmc_run(tmp_path / "a", [(1, ours, "MfmaFlopsBF16", 2e9, 1000), (1, ours, "GRBM_GUI_ACTIVE", 8 * 2000, 1000),
                              (2, ours, "MfmaFlopsBF16", 4e9, 2000), (2, ours, "GRBM_GUI_ACTIVE", 8 * 4000, 2000),
                              (3, vend, "MfmaFlopsBF16", 2e9, 800), (3, vend, "GRBM_GUI_ACTIVE", 8 * 1600, 800),
                              (4, other, "MfmaFlopsBF16", 0, 10)])
    _pmc_run(tmp_path / "b", [(1, ours, "SQ_WAIT_ANY", 10, 1000), (2, ours, "SQ_WAIT_ANY", 30, 2000),
                              (3, vend, "SQ_WAIT_ANY", 5, 800)])
    bench.pmc_summary([str(tmp_path / "a"), str(tmp_path / "b")])
    out = capsys.readouterr().out.splitlines()
    hdr = [h.strip() for h in out[0].strip("|").split("|")]
    rows = [dict(zip(hdr, [c.strip() for c in line.strip("|").split("|")])) for line in out[2:]]
    assert len(rows) == 3
    by = {(r["kernel"], r["GFLOP"]): r for r in rows}
    a = by[("`gemm4_bf16_nt_kernel<8, 8, true, false, 0>`", "2.0")]
    b = by[("`gemm4_bf16_nt_kernel<8, 8, true, false, 0>`", "4.0")]
    v = by[("`hipBLASLt MT256x256x64 stream-K`", "2.0")]
    assert a["SQ_WAIT_ANY"] == "10" and b["SQ_WAIT_ANY"] == "30" and v["SQ_WAIT_ANY"] == "5"
    # clock = GUI-active cycles per XCD over the dispatch time: 2000 cycles in 1 us = 2 GHz
    assert a["clock GHz"] == "2" and b["clock GHz"] == "2" and v["clock GHz"] == "2"
    assert a["dispatches"] == "1"
