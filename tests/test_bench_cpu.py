"""Host logic of bench.py (no GPU): the one-GPU refusal, the code digest that keys committed counter
summaries, and the traffic figures computed from rocprofv3 counter CSVs."""
import csv
import importlib.util
import json
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    for extra, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})):
        p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *extra], capture_output=True, text=True,
                           env={**os.environ, **env}, timeout=120)
        assert p.returncode == 2
        assert "one GPU" in p.stderr and p.stdout == ""


def test_code_digest_ignores_comments_and_layout(bench):
    a = "int f(int x) { // the sum\n  return x + 1; /* one */ }"
    b = "int f(int x)   {\n\n return x + 1;   }"
    c = "int f(int x) { return x + 2; }"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)
    d = bench.source_digest("nf4_gemv")
    assert len(d) == 16 and d == bench.source_digest("nf4_gemv")
    assert d != bench.source_digest("nf4_gemm_fwd")


FIELDS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
          "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
          "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _counter_csv(path, counter, rows):
    """rows: (dispatch id, kernel name, value in KiB); a dispatch may appear on several rows (per-XCD
    values), which the bench adds."""
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, FIELDS)
        w.writeheader()
        for disp, name, kib in rows:
            w.writerow({**{k: 0 for k in FIELDS}, "Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": kib})


def test_traffic_from_counter_runs(bench, tmp_path, monkeypatch):
    d = tmp_path / "counters"
    cal_kib = (256 << 20) / 1024
    # the copy's FETCH_SIZE reads half its bytes (scale 2), WRITE_SIZE all of them (scale 1)
    _counter_csv(str(d / "calib_fetch"), "FETCH_SIZE", [(1, "__amd_rocclr_copyBuffer", cal_kib / 2)])
    _counter_csv(str(d / "calib_write"), "WRITE_SIZE", [(1, "__amd_rocclr_copyBuffer", cal_kib)])
    gemv = "void qlora::k_nf4_gemv_m32<1>(unsigned short const*, long)"
    other = "void qlora::k_gemv_finish<2, 16>(float const*)"
    _counter_csv(str(d / "fetch"), "FETCH_SIZE", [(5, gemv, 100.0), (5, gemv, 50.0), (6, gemv, 250.0), (7, other, 9e6)])
    _counter_csv(str(d / "write"), "WRITE_SIZE", [(5, gemv, 10.0), (6, gemv, 30.0), (7, other, 9e6)])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "traffic_path", lambda k, wl: str(out))
    args = types.SimpleNamespace(traffic_from=str(d), traffic_command="cmd")
    bench.write_traffic(args, "wl", ["nf4_gemv"])
    t = json.loads(out.read_text())
    assert t["dispatches"] == [2, 2]
    assert t["fetch_scale"] == pytest.approx(2.0) and t["write_scale"] == pytest.approx(1.0)
    assert t["fetch_bytes_per_launch"] == pytest.approx((150.0 + 250.0) / 2 * 1024 * 2.0)
    assert t["write_bytes_per_launch"] == pytest.approx((10.0 + 30.0) / 2 * 1024)
    assert t["hbm_bytes_per_launch"] == pytest.approx(t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"])
    assert t["source_digest"] == bench.source_digest("nf4_gemv")
    # a committed summary counts only while the kernel's code is the one it was taken from
    monkeypatch.setattr(bench, "traffic_path", lambda k, wl: str(out))
    assert bench.traffic_from_profiles("nf4_gemv", "wl") == pytest.approx(t["hbm_bytes_per_launch"])
    t["source_digest"] = "0" * 16
    out.write_text(json.dumps(t))
    assert bench.traffic_from_profiles("nf4_gemv", "wl") is None
