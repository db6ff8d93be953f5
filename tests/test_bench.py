"""bench.py host logic on the CPU: the one-GPU guard, and the traffic
bookkeeping that turns rocprofv3 FETCH_SIZE / WRITE_SIZE runs into bytes per
launch (fed here with hand-made counter files)."""
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
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _write_run(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for disp, kernel, value in rows:
            # two counter instances per dispatch: the reader must add them up
            w.writerow([disp, kernel, counter, value / 2])
            w.writerow([disp, kernel, counter, value / 2])


def test_traffic_is_scaled_by_the_copy_and_skips_the_warmup(tmp_path):
    prof = tmp_path / "prof"
    gib_kib = float(1 << 20)
    # the copy of 1 GiB reads as half of it (factor 2) and writes as all of it
    _write_run(prof / "fetch_copy", "FETCH_SIZE", [(1, "fill", 7.0), (2, "__amd_rocclr_copyBuffer", gib_kib / 2)])
    _write_run(prof / "write_copy", "WRITE_SIZE", [(2, "__amd_rocclr_copyBuffer", gib_kib)])
    k = "void qgemm::qgemm_dma_kernel<0, 4, 4, 2, true, 1, 0>(qgemm::Params)"
    _write_run(prof / "fetch_w", "FETCH_SIZE", [(3, k, 999.0), (4, k, 100.0), (5, k, 300.0)])
    _write_run(prof / "write_w", "WRITE_SIZE", [(3, k, 50.0), (4, k, 60.0)])
    out = tmp_path / "traffic.json"
    t = bench.write_traffic(str(prof), ["w"], out_path=str(out))
    assert t["copy_factor"] == {"FETCH_SIZE": 2.0, "WRITE_SIZE": 1.0}
    assert t["workloads"]["w"]["fetch_bytes"] == round((100 + 300) / 2 * 1024 * 2.0)
    assert t["workloads"]["w"]["write_bytes"] == round(60 * 1024)
    assert json.load(open(out))["kernel_sha256"] == bench.kernel_digest()


def test_kernel_digest_is_stable_hex():
    a, b = bench.kernel_digest(), bench.kernel_digest()
    assert a == b and len(a) == 64
    int(a, 16)
