"""Host logic of bench.py that needs no GPU: the counter summary that turns
two rocprofv3 --pmc runs into per-launch HBM bytes, and the refusal of
multi-GPU runs."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

HEADER = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
          "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
          "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _write_run(d, counter, rows):
    """rows: (dispatch id, kernel name, counter value in KiB)."""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "bench_counter_collection.csv"), "w", newline="") as fh:
        w = csv.writer(fh, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(HEADER)
        for i, name, val in rows:
            w.writerow([i, i, "Agent 1", 1, 1, 1, 256, 1, name, 256, 0, 0, 16, 0, 16, counter, val, 0, 1])


def test_traffic_summary_calibrates_and_takes_medians(tmp_path):
    slow = "void sfi::slow_partial_kernel<sfi::BF16, 128, 4>(sfi::SlowArgs)"
    gather = "sfi::select_gather_kernel(sfi::SelectArgs)"
    copy = "void at::native::vectorized_elementwise_kernel<4, copy>(int)"
    # FETCH_SIZE reads half of a copy's bytes (factor 2), WRITE_SIZE all of them (factor 1)
    fetch = [(1, "void at::native::randn_kernel()", 5.0), (2, slow, 100.0), (3, slow, 300.0), (4, slow, 200.0),
             (5, gather, 10.0), (6, copy, 4.0 * 1024)]
    write = [(1, slow, 50.0), (2, slow, 70.0), (3, gather, 1.0), (4, copy, 8.0 * 1024)]
    _write_run(str(tmp_path / "fetch"), "FETCH_SIZE", fetch)
    _write_run(str(tmp_path / "write"), "WRITE_SIZE", write)
    out = tmp_path / "traffic.json"
    t = bench.traffic_summary(str(tmp_path / "fetch"), str(tmp_path / "write"), 8, str(out))
    assert json.loads(out.read_text()) == t
    assert t["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert t["calibration"]["write_factor"] == pytest.approx(1.0)
    k = t["kernels"]
    assert set(k) == {"sfi::slow_partial_kernel<sfi::BF16, 128, 4>(sfi::SlowArgs)", gather}
    s = k["sfi::slow_partial_kernel<sfi::BF16, 128, 4>(sfi::SlowArgs)"]
    assert s["group"] == "slow_partial" and s["dispatches_fetch"] == 3 and s["dispatches_write"] == 2
    assert s["fetch_bytes"] == pytest.approx(200.0 * 1024 * 2)   # median of 100, 300, 200 KiB, scaled
    assert s["write_bytes"] == pytest.approx(60.0 * 1024)        # median of 50 and 70 KiB
    assert k[gather]["group"] == "select"
    assert t["csrc_digest"] == bench.csrc_digest()


def test_digest_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    src = tmp_path / "sparse_kv_attention_sfi_amd" / "csrc"
    src.mkdir(parents=True)
    f = src / "k.hip"
    f.write_text("int a = 1; // one\n/* block */ int b;\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    d0 = bench.csrc_digest()
    f.write_text("int a = 1;   // changed comment\n\n int b;")
    assert bench.csrc_digest() == d0
    f.write_text("int a = 2; int b;")
    assert bench.csrc_digest() != d0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def test_traffic_rate():
    r = bench.traffic_rate(4e9, 1e3)           # 4 GB in 1 ms
    assert r["traffic_GBps"] == pytest.approx(4000.0)
    assert r["traffic_frac"] == pytest.approx(4000.0 / bench.HBM_PEAK_GBS)
    assert bench.traffic_rate(None, 5.0) == {}
