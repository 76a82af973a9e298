"""Host-side parts of bench.py: the single-GPU guard and the rocprofv3
post-processing that writes the profiles/ summaries (CPU only)."""

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
          "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
          "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
FWD = "_ZN2fa12_GLOBAL__N_120attn_fwd_pipe_kernelIDF16bLi128ELi0ELb1ELb0EEEvNS0_9FwdParamsE"
COPY = "void at::native::elementwise_kernel<neg>"


def _write(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for disp, name, counter, value, t0, t1 in rows:
            w.writerow({k: 0 for k in FIELDS} | {"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": counter,
                                                 "Counter_Value": value, "Start_Timestamp": t0,
                                                 "End_Timestamp": t1})


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_summary_scales_by_the_copy(tmp_path, monkeypatch):
    """Each counter is averaged over the dispatches after the first and
    scaled by what it reads for the calibration copy of COPY_BYTES."""
    kib = bench.COPY_BYTES / 1024
    # the copy reads half its bytes on FETCH_SIZE (scale 2) and all on WRITE_SIZE (scale 1)
    _write(str(tmp_path / "f" / "fetch_counter_collection.csv"),
           [(1, FWD, "FETCH_SIZE", 999.0, 0, 1), (2, FWD, "FETCH_SIZE", 100.0, 0, 1), (3, FWD, "FETCH_SIZE", 300.0, 0, 1),
            (4, COPY, "FETCH_SIZE", kib / 2, 0, 1)])
    _write(str(tmp_path / "w" / "write_counter_collection.csv"),
           [(1, FWD, "WRITE_SIZE", 7.0, 0, 1), (2, FWD, "WRITE_SIZE", 50.0, 0, 1), (3, FWD, "WRITE_SIZE", 50.0, 0, 1),
            (4, COPY, "WRITE_SIZE", kib, 0, 1)])
    os.makedirs(tmp_path / "profiles")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_digest", lambda paths: "digest")
    bench.summarize_traffic(str(tmp_path / "f"), str(tmp_path / "w"))
    with open(tmp_path / "profiles" / "traffic.json") as f:
        rec = json.load(f)["causal_bf16_b4h16_s2048_d128"]["fwd"]
    assert rec["fetch_kib"] == 200.0 and rec["write_kib"] == 50.0
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    assert rec["bytes_per_launch"] == round(200.0 * 1024 * 2 + 50.0 * 1024)
    assert rec["source_digest"] == "digest"


def test_counter_summary_derives_clock_and_mfma_busy(tmp_path, capsys):
    """GPU cycles = GRBM_GUI_ACTIVE / 8 XCDs; MFMA busy = busy cycles over
    cycles x 1024 SIMDs; the clock is cycles over the dispatch duration."""
    cycles = 100000
    rows = []
    for disp in (1, 2, 3):
        rows.append((disp, FWD, "GRBM_GUI_ACTIVE", 8 * cycles, 0, 50000))           # 50 us
        rows.append((disp, FWD, "SQ_VALU_MFMA_BUSY_CYCLES", 0.25 * cycles * 1024, 0, 50000))
    _write(str(tmp_path / "p" / "pmc_counter_collection.csv"), rows)
    bench.summarize_counters([str(tmp_path / "p")])
    out = capsys.readouterr().out
    assert "| (derived) GPU cycles per dispatch | 100000 |" in out
    assert "| (derived) shader clock, GHz (cycles / dispatch duration) | 2.000 |" in out
    assert "| (derived) MFMA busy, share of SIMD-cycles | 0.2500 |" in out
