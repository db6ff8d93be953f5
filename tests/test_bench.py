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


def _shape_only(name):
    """A workload dict with arrays of the recipe's shapes and dtypes (no
    random draws): enough for the byte bookkeeping."""
    import numpy as np
    from block_scaled_precision_02_amd import inputs
    kind, M, N, K, _, has_bias, fmt, brows = inputs.WORKLOADS[name]
    d = dict(name=name, kind=kind, fmt=fmt, M=M, N=N, K=K, b_rows_per_scale=brows)
    fa, fb = (fmt.split("/") if fmt and "/" in fmt else (fmt, fmt))
    d["A"] = np.empty((M, K // 2 if fa == "e2m1" else K), np.uint8)
    d["B"] = np.empty((N, K // 2 if fb == "e2m1" else K), np.uint8)
    if kind == "mx":
        d["scale_a"] = np.empty((M, K // 32), np.uint8)
        d["scale_b"] = np.empty((-(-N // brows), K // 32), np.uint8)
    else:
        d["scale_a"] = np.empty(M, np.float32)
        d["scale_b"] = np.empty(N, np.float32)
    d["bias"] = np.empty(N, np.uint16) if has_bias else None
    return d


def test_cold_rotation_counts_exceed_twice_the_mall():
    """R = ceil(512 MB / operand bytes): 12, 11, 8, 2 input sets for the FP8,
    MXFP8, MXFP4 and large INT8 workloads; the latency-bound INT8 256^3-class
    workload runs on one set."""
    want = {"i8_small": 1, "f8_ptpc": 12, "mxfp8": 11, "mxfp4": 8, "i8_qkv": 2}
    for _, name in bench.SUITE:
        d = _shape_only(name)
        R = bench.cold_sets(d)
        assert R == want[name], (name, R)
        if R > 1:
            assert R * bench.operand_bytes(d) >= 512e6 > (R - 1) * bench.operand_bytes(d)


def test_sample_rows_cover_both_ends():
    import numpy as np
    r = bench.sample_rows(30000)
    assert r[0] == 0 and r[1] == 1 and r[-1] == 29999 and r[-2] == 29998
    assert len(r) == 16 and np.all(np.diff(r) > 0)
    assert list(bench.sample_rows(5)) == [0, 1, 2, 3, 4]


def test_pass_stats():
    s = bench.pass_stats([2.0, 1.0, 4.0], 2e12, 1000.0)
    assert s["ms_median"] == 2.0 and s["ms_min"] == 1.0 and s["spread"] == 1.5
    assert s["rate"] == 1000.0 and s["rate_best"] == 2000.0 and s["frac"] == 1.0


def test_clock_sampler_reads_the_starred_level(tmp_path):
    f = tmp_path / "pp_dpm_sclk"
    f.write_text("0: 500Mhz\n1: 1712Mhz *\n2: 2400Mhz\n")
    c = bench.ClockSampler()
    c.path = str(f)
    assert c.read() == 1712.0
    c.path = str(tmp_path / "missing")
    assert c.read() is None
