"""Benchmark of the scaled low-precision GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]          # the five workloads
    python bench.py --workload NAME [--shape M,N,K] [--tile T]   # one workload

A step is one call of the GEMM (argument checks, tile choice, one kernel:
tile schedule, HBM->LDS staging, MFMA K loop, fused scale/bias epilogue) on
one batch of seeded synthetic inputs already resident in HBM.

Default run.  The headline (`value`, `ms_per_step`, `roofline`) is the INT8
rowwise projection M=30000 N=21504 K=5376 with bias: W warmup steps, then
exactly K timed steps between two device synchronisations.  The same line
carries `per_config`: each of the five workloads (INT8 256x256x512, FP8
per-token 4096x2112x7168, MXFP8 16384x7168x2048, MXFP4 8192^3, INT8
30000x21504x5376) timed cold -- R input sets at distinct device addresses,
R = ceil(512 MB / operand bytes) so that the operands cannot be served from
the 256 MB MALL or L2 -- in 3 passes of >= 100 ms (median, min, spread),
with the shader clock sampled during the passes, a hot (one input set)
secondary, the prepacked-B entry point, and a parity verdict on sampled
output rows against the CPU oracle.  The oracle also gives the CPU baseline
(a bounded sample of the headline workload on this host's cores).

--workload picks one workload instead (i8_small, f8_ptpc, mxfp8, mxfp4,
i8_qkv, f8_block: FP8 with fp32 scales per 128-element K block,
16384x7168x2048; mx_a8w4 / mx_a4w8: MX e4m3 A x e2m1 B and e2m1 A x e4m3 B,
8192^3; mxfp6 / mxfp6_e3m2: MX
with the 6-bit E2M3 / E3M2 elements, 8192^3).
"""
import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective TFLOPS/TOPS (2MNK/t) per dtype; % of MI355X dense MFMA peak"
# MI355X dense matrix-core peaks (TOPS / TFLOPS) and HBM bandwidth (GB/s)
# (mixed e4m3 / e2m1 MX runs at the e4m3 rate: the scaled MFMA takes 64
# cycles when either operand is 8-bit)
PEAK = {"i8": 5000.0, "f8": 5000.0, "f8b": 5000.0, "e4m3": 5000.0, "e2m1": 10100.0, "e4m3/e2m1": 5000.0,
        "e2m1/e4m3": 5000.0, "e2m3": 10100.0, "e3m2": 10100.0}
HBM_GBPS = 8000.0
# The pages' numbers for exactly these workloads (2MNK / their time where they
# give a time); context, not targets:
#  - MXFP8 16384x7168x2048: 246.2 us and 32768x7168x1792: 462.2 us, FP8
#    blockscale 16384x7168x2048: 362.3 us, all on MI355X (ROCm/mori PR #806,
#    commit message table; its MXFP8 reads a packed scale layout);
#  - MXFP4 8192^3: 5034 TFLOPS on MI355X with a preshuffled B (ROCm/FlyDSL PR
#    #990, Performance), so it is set against the prepacked-B call.
# vs_baseline divides by one of these only when the pages measured MI355X.
PAGES_REF = {
    ("mxfp8", 16384, 7168, 2048): 2.0 * 16384 * 7168 * 2048 / 246.2e-6 / 1e12,
    ("mxfp8", 32768, 7168, 1792): 2.0 * 32768 * 7168 * 1792 / 462.2e-6 / 1e12,
    ("f8_block", 16384, 7168, 2048): 2.0 * 16384 * 7168 * 2048 / 362.3e-6 / 1e12,
}
PAGES_REF_PREPACKED = {("mxfp4", 8192, 8192, 8192): 5034.0}
# The one number the pages give for the INT8 workload was measured on another
# GPU (RX 9070 XT, gfx1201; comfy-kitchen PR #174, Performance): reported as
# context, never divided into an MI355X rate.
PAGES_CONTEXT = {("i8_qkv", 30000, 21504, 5376): {"value": 209.9, "unit": "TOPS", "hardware": "RX 9070 XT (gfx1201)",
                                                  "source": "comfy-kitchen PR #174, Performance"}}
# Cold timing: R input sets at distinct device addresses, R = ceil(512 MB /
# operand bytes), twice the 256 MB MALL, so no launch finds its operands in
# the MALL or L2 from an earlier one (FP8 4096x2112x7168: 12, MXFP8
# 16384x7168x2048: 11, MXFP4 8192^3: 8, INT8 30000x21504x5376: 2).  The INT8
# 256x256x512 workload is launch-latency bound and runs on one set.
COLD_BYTES = 512e6
LATENCY_BOUND = {"i8_small"}
SUITE = [(1, "i8_small"), (2, "f8_ptpc"), (3, "mxfp8"), (4, "mxfp4"), (5, "i8_qkv")]
HEADLINE = "i8_qkv"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dtype_of(d):
    return d["kind"] if d["kind"] != "mx" else d["fmt"]


def unit_of(d):
    return "TOPS" if d["kind"] == "i8" else "TFLOPS"


MX_FMT = {"e4m3": 0, "e2m1": 1, "e2m3": 2, "e3m2": 3}
ROW_BYTES = {"e4m3": lambda K: K, "e2m1": lambda K: K // 2, "e2m3": lambda K: 3 * K // 4, "e3m2": lambda K: 3 * K // 4}


class Launcher:
    """Binds one workload's device buffers to a direct C-ABI call (the
    binding's argument checks are done once, outside the timed loop)."""

    def __init__(self, d, sets, out, stream, prepacked=False):
        import block_scaled_precision_02_amd as q
        self.L = q.lib()
        self.d = d
        self.sets = sets
        self.out = out
        self.stream = ctypes.c_void_p(stream)
        N = d["N"]
        self.ldc = out.stride(0)
        self.args = []
        for s in sets:
            bias = None if s["bias"] is None else s["bias"].data_ptr()
            if prepacked and "/" in (d["fmt"] or ""):
                # e2m1 B: the 32-row packer; e4m3 B (under e2m1 A): the 16-row one
                a4 = d["fmt"] == "e2m1/e4m3"
                pb = (q.qgemm_prepack_b(s["B"]) if a4 else q.qgemm_prepack_b32(s["B"])).data
                s["Bp"] = pb
                a = ((1, 0) if a4 else (0, 1)) + (s["A"].data_ptr(), s["A"].stride(0), pb.data_ptr(), s["scale_a"].data_ptr(),
                     s["scale_b"].data_ptr(), d["b_rows_per_scale"], bias, out.data_ptr(), self.ldc, d["M"], N, d["K"],
                     self.stream)
                self.args.append((self.L.qgemm_mx_mixed_prepacked, a))
                continue
            if prepacked:
                # B prepacked once, outside the timed region (the weights are static)
                pb = q.qgemm_prepack_b(s["B"]).data
                s["Bp"] = pb
                if d["kind"] == "i8":
                    a = (s["A"].data_ptr(), s["A"].stride(0), pb.data_ptr(), s["scale_a"].data_ptr(),
                         s["scale_b"].data_ptr(), bias, out.data_ptr(), self.ldc, d["M"], N, d["K"], self.stream)
                    self.args.append((self.L.qgemm_i8_rowwise_prepacked, a))
                elif d["kind"] in ("f8", "f8b"):
                    a = (s["A"].data_ptr(), s["A"].stride(0), pb.data_ptr(), s["scale_a"].data_ptr(),
                         s["scale_b"].data_ptr(), bias, out.data_ptr(), self.ldc, d["M"], N, d["K"], self.stream)
                    fn = self.L.qgemm_f8_pertoken_prepacked if d["kind"] == "f8" else self.L.qgemm_f8_blockscale_prepacked
                    self.args.append((fn, a))
                else:
                    fmt = MX_FMT[d["fmt"]]
                    a = (fmt, s["A"].data_ptr(), s["A"].stride(0), pb.data_ptr(), s["scale_a"].data_ptr(),
                         s["scale_b"].data_ptr(), d["b_rows_per_scale"], bias, out.data_ptr(), self.ldc, d["M"], N,
                         d["K"], self.stream)
                    self.args.append((self.L.qgemm_mx_prepacked, a))
                continue
            if d["kind"] == "i8":
                a = (s["A"].data_ptr(), s["A"].stride(0), s["B"].data_ptr(), s["B"].stride(0),
                     s["scale_a"].data_ptr(), s["scale_b"].data_ptr(), bias, out.data_ptr(),
                     self.ldc, d["M"], N, d["K"], self.stream)
                self.args.append((self.L.qgemm_i8_rowwise, a))
            elif d["kind"] == "f8":
                a = (s["A"].data_ptr(), s["A"].stride(0), s["B"].data_ptr(), s["B"].stride(0),
                     s["scale_a"].data_ptr(), s["scale_b"].data_ptr(), bias, out.data_ptr(),
                     self.ldc, d["M"], N, d["K"], self.stream)
                self.args.append((self.L.qgemm_f8_pertoken, a))
            elif d["kind"] == "f8b":
                a = (s["A"].data_ptr(), s["A"].stride(0), s["B"].data_ptr(), s["B"].stride(0),
                     s["scale_a"].data_ptr(), s["scale_b"].data_ptr(), bias, out.data_ptr(),
                     self.ldc, d["M"], N, d["K"], self.stream)
                self.args.append((self.L.qgemm_f8_blockscale, a))
            elif "/" in d["fmt"]:
                fa, fb = (0 if f == "e4m3" else 1 for f in d["fmt"].split("/"))
                a = (fa, fb, s["A"].data_ptr(), s["A"].stride(0), s["B"].data_ptr(), s["B"].stride(0),
                     s["scale_a"].data_ptr(), s["scale_b"].data_ptr(), d["b_rows_per_scale"], bias,
                     out.data_ptr(), self.ldc, d["M"], N, d["K"], self.stream)
                self.args.append((self.L.qgemm_mx_mixed, a))
            else:
                fmt = MX_FMT[d["fmt"]]
                a = (fmt, s["A"].data_ptr(), s["A"].stride(0), s["B"].data_ptr(), s["B"].stride(0),
                     s["scale_a"].data_ptr(), s["scale_b"].data_ptr(), d["b_rows_per_scale"], bias,
                     out.data_ptr(), self.ldc, d["M"], N, d["K"], self.stream)
                self.args.append((self.L.qgemm_mx, a))

    def __call__(self, i):
        fn, a = self.args[i % len(self.args)]
        st = fn(*a)
        if st != 0:
            raise RuntimeError(self.L.qgemm_last_error().decode())


def upload(d):
    import torch
    t = {}
    for k in ("A", "B", "scale_a", "scale_b"):
        t[k] = torch.from_numpy(np.ascontiguousarray(d[k])).cuda()
    t["bias"] = None if d["bias"] is None else torch.from_numpy(d["bias"].view(np.int16)).cuda()
    return t


KERNEL_SOURCES = "block_scaled_precision_02_amd/csrc"
# workloads whose FETCH_SIZE / WRITE_SIZE runs profiles/traffic.json holds
TRAFFIC_WORKLOADS = ["i8_qkv", "mxfp4", "f8_ptpc", "mxfp8", "mxfp6", "f8_block", "mx_a8w4", "mx_a4w8"]
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_digest():
    """sha256 over the GEMM's kernel source files (name and bytes, sorted by
    name); the activation quantisers' and the B prepacking's own files are
    not part of it."""
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, KERNEL_SOURCES)
    for n in sorted(os.listdir(d)):
        if n.endswith((".hip", ".hpp", ".cpp", ".h")) and not n.startswith(("qgemm_quant", "qgemm_pack")):
            h.update(n.encode())
            h.update(open(os.path.join(d, n), "rb").read())
    return h.hexdigest()


def min_bytes(d):
    """Algorithmic HBM bytes of one call: A, B, C and the scale / bias arrays,
    each read or written once."""
    M, N, K = d["M"], d["N"], d["K"]
    fmts = (d.get("fmt") or "").split("/")
    fa, fb = (fmts[0], fmts[-1]) if fmts[0] else (None, None)
    ab = M * (ROW_BYTES[fa](K) if fa else K) + N * (ROW_BYTES[fb](K) if fb else K)
    if d["kind"] == "mx":
        sc = M * (K // 32) + (-(-N // d["b_rows_per_scale"])) * (K // 32)
    elif d["kind"] == "f8b":
        sc = 4 * (M + (-(-N // 128))) * (K // 128)
    else:
        sc = 4 * (M + N)
    return ab + sc + 2 * M * N + (2 * N if d["bias"] is not None else 0)


def traffic_bytes(name):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary, already scaled by the copy-kernel factors; None when the kernel
    sources have changed since those counters were taken."""
    try:
        t = json.load(open(TRAFFIC_JSON))
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha256") != kernel_digest():
        return None
    w = t.get("workloads", {}).get(name)
    return None if w is None else w["fetch_bytes"] + w["write_bytes"]


def _counter_per_dispatch(csv_path, counter, kernel_substr):
    import csv
    import collections
    agg = collections.defaultdict(float)
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] == counter and kernel_substr in r["Kernel_Name"]:
            agg[int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    return [agg[d] for d in sorted(agg)]


def write_traffic(prof_dir, workloads, out_path=TRAFFIC_JSON):
    """Build profiles/traffic.json from rocprofv3 --pmc runs laid out as
    <prof_dir>/{fetch,write}_<name>/run_counter_collection.csv, <name> being
    each workload and "copy" (bench.py --copy-bytes 1 GiB, the calibration).
    Counters are KiB per dispatch; the timed dispatches are all but the first
    (warmup) one of each run; the copy factor is 1 GiB over what the counter
    reads for the copy."""
    out = {"kernel_sources": KERNEL_SOURCES, "kernel_sha256": kernel_digest(), "copy_factor": {},
           "workloads": {}, "unit": "bytes per launch"}
    for what, counter in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        copy = _counter_per_dispatch(os.path.join(prof_dir, f"{what}_copy", "run_counter_collection.csv"),
                                     counter, "copyBuffer")
        factor = float(1 << 30) / (copy[-1] * 1024.0)
        out["copy_factor"][counter] = round(factor, 4)
        for name in workloads:
            v = _counter_per_dispatch(os.path.join(prof_dir, f"{what}_{name}", "run_counter_collection.csv"),
                                      counter, "qgemm")
            v = v[1:] if len(v) > 1 else v
            out["workloads"].setdefault(name, {})[f"{what}_bytes"] = round(sum(v) / len(v) * 1024.0 * factor)
    with open(out_path, "w") as fh:
        json.dump(out, fh, indent=1)
    return out


def cpu_baseline(d, target_s):
    """The oracle, as it is, on whole rows of the same workload: a few rows
    first to calibrate, then enough rows for about target_s seconds.  The
    calibration takes two rows per oracle thread, so that it runs on all of
    them as the timed sample does (two rows alone ran on two threads, and the
    sample came out several times shorter than target_s)."""
    import oracle
    from tests import parity
    rows = np.arange(min(2 * oracle.num_threads(), d["M"]))
    t0 = time.perf_counter()
    parity.oracle_run(d, rows=rows)
    t1 = time.perf_counter() - t0
    per_row = max(t1 / len(rows), 1e-6)
    n = int(min(d["M"], max(len(rows), target_s / per_row)))
    rows = np.linspace(0, d["M"] - 1, n).astype(np.int64)
    t0 = time.perf_counter()
    parity.oracle_run(d, rows=rows)
    t = time.perf_counter() - t0
    ops = 2.0 * n * d["N"] * d["K"]
    return {"value": round(ops / t / 1e12, 6), "unit": unit_of(d), "cores": oracle.num_threads(),
            "kind": "oracle", "host": host_info(),
            "sample": f"{n} of {d['M']} rows of A (all {d['N']} columns, K={d['K']}), {t:.1f} s"}


def bench_quant(args):
    """The activation quantiser on the A operand shape of a GEMM workload:
    HBM-bound, so the rate is algorithmic bytes (bf16 in, codes and scales
    out) over the kernel time, against the HBM peak."""
    import torch
    from block_scaled_precision_02_amd import inputs
    import block_scaled_precision_02_amd as q

    wl, M, K = inputs.QUANT_SHAPES[args.quant]
    R = args.rot or 4          # 4 x 58-268 MB of activations: past the 256 MB MALL
    log(f"[bench] quantiser {args.quant} M={M} K={K} x{R}")
    xs = [torch.from_numpy(inputs.make_activations(M, K, rot=r).view(np.int16)).cuda() for r in range(R)]
    L = q.lib()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    if args.quant == "f8":
        Q = torch.empty((M, K), dtype=torch.uint8, device="cuda")
        S = torch.empty(M, dtype=torch.float32, device="cuda")
        nbytes = 2 * M * K + M * K + 4 * M

        def run(i):
            return L.qgemm_quant_f8_pertoken(xs[i % R].data_ptr(), K, Q.data_ptr(), K, S.data_ptr(), M, K, sp)
        dtype = "bf16->e4m3"
    elif args.quant == "f8_block":
        Q = torch.empty((M, K), dtype=torch.uint8, device="cuda")
        S = torch.empty((M, K // 128), dtype=torch.float32, device="cuda")
        nbytes = 2 * M * K + M * K + 4 * M * (K // 128)

        def run(i):
            return L.qgemm_quant_f8_block(xs[i % R].data_ptr(), K, Q.data_ptr(), K, S.data_ptr(), K // 128, M, K, sp)
        dtype = "bf16->e4m3 (1x128 blocks)"
    else:
        fmt = 0 if args.quant == "mxfp8" else 1
        row = K if fmt == 0 else K // 2
        Q = torch.empty((M, row), dtype=torch.uint8, device="cuda")
        S = torch.empty((M, K // 32), dtype=torch.uint8, device="cuda")
        nbytes = 2 * M * K + M * row + M * (K // 32)

        def run(i):
            return L.qgemm_quant_mx(fmt, xs[i % R].data_ptr(), K, Q.data_ptr(), row, S.data_ptr(), K // 32, M, K,
                                    sp)
        dtype = "bf16->mx-" + ("e4m3" if fmt == 0 else "e2m1")
    for i in range(args.warmup):
        if run(i) != 0:
            raise RuntimeError(L.qgemm_last_error().decode())
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        run(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = ev0.elapsed_time(ev1) / args.steps
    gbps = nbytes / (kernel_ms * 1e-3) / 1e9
    res = {"metric": "activation quantiser HBM rate (algorithmic bytes / kernel time)",
           "value": round(nbytes / (wall / args.steps) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 6),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
           "data": "synthetic",
           "config": {"workload": f"quant {args.quant} M={M} K={K} (A of {wl})", "rotating_sets": R},
           "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_GBPS, "unit": "GB/s",
                        "frac": round(gbps / HBM_GBPS, 4), "traffic": None, "kernel_ms": round(kernel_ms, 6),
                        "algorithmic_bytes": nbytes},
           "cpu_baseline": None}
    if not args.no_cpu_baseline:
        import oracle
        X = inputs.make_activations(M, K)
        rows = max(1, min(M, int(M * 0.25)))
        t0 = time.perf_counter()
        if args.quant == "f8":
            oracle.quant_f8_pertoken(X[:rows])
        elif args.quant == "f8_block":
            oracle.quant_f8_block(X[:rows])
        else:
            oracle.quant_mx(0 if args.quant == "mxfp8" else 1, X[:rows])
        t = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(nbytes * rows / M / t / 1e9, 3), "unit": "GB/s",
                               "cores": oracle.num_threads(), "kind": "oracle",
                               "sample": f"{rows} of {M} rows"}
    return res


def time_graph(d, sets, out, args):
    """args.graph calls (cycling over the input sets) captured in one HIP graph
    on a side stream, replayed; per-call time = replay time / calls.  Every
    replay's output must equal the eager call's on the same last input set."""
    import torch
    n = args.graph
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    run = Launcher(d, sets, out, side.cuda_stream, prepacked=args.prepacked)
    with torch.cuda.stream(side):
        run(n - 1)                                   # eager: the graph's last call, same inputs
    side.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for i in range(n):
            run(i)
    replays = max(3, args.steps // n)
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(out, eager):
            raise RuntimeError("graph replay output differs from the eager call")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    ev0.record(stream)
    for _ in range(replays):
        g.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / (replays * n)
    return {"calls_per_graph": n, "replays": replays, "ms_per_call": round(ms, 6),
            "rate": round(2.0 * d["M"] * d["N"] * d["K"] / (ms * 1e-3) / 1e12, 3)}


def operand_bytes(d):
    """Bytes of one input set: A, B, the scale arrays and the bias."""
    n = 0
    for k in ("A", "B", "scale_a", "scale_b", "bias"):
        if d.get(k) is not None:
            n += np.asarray(d[k]).nbytes
    return n


def cold_sets(d):
    return 1 if d["name"] in LATENCY_BOUND else max(2, -(-int(COLD_BYTES) // operand_bytes(d)))


def make_sets(d0, R):
    """Set 0 uploaded from the generator, sets 1..R-1 device copies of it at
    distinct addresses (the caches key on addresses, not on values)."""
    s0 = upload(d0)
    sets = [s0]
    for _ in range(1, R):
        sets.append({k: (None if v is None else v.clone()) for k, v in s0.items()})
    return sets


class ClockSampler:
    """Samples the shader clock the driver reports (the starred level of
    pp_dpm_sclk, which on this part reads the current frequency) every
    `period` seconds from a thread while a timed region runs.  None where
    the file does not exist."""

    def __init__(self, period=0.02):
        import glob
        import threading
        f = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.path = f[0] if f else None
        self.period = period
        self.samples = []
        self._stop = threading.Event()
        self._thread = None

    def read(self):
        if self.path is None:
            return None
        try:
            for line in open(self.path):
                if "*" in line:
                    return float(line.split(":")[1].strip().rstrip("*").strip().lower().replace("mhz", ""))
        except (OSError, ValueError, IndexError):
            return None
        return None

    def __enter__(self):
        import threading
        if self.path is not None:
            def loop():
                while not self._stop.is_set():
                    v = self.read()
                    if v is not None:
                        self.samples.append(v)
                    self._stop.wait(self.period)
            self._thread = threading.Thread(target=loop, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()

    def summary(self, min_samples=10):
        """Median, min and max of the samples; None when fewer than
        `min_samples` were taken (a region too short for the driver's
        reading to have settled)."""
        if len(self.samples) < min_samples:
            return None
        v = np.array(self.samples)
        return {"median": float(np.median(v)), "min": float(v.min()), "max": float(v.max()), "samples": len(v)}


def gpu_busy_percent(samples=5, period=0.02):
    """The driver's busy figure before a timed region (idle check), or None."""
    import glob
    f = sorted(glob.glob("/sys/class/drm/card*/device/gpu_busy_percent"))
    if not f:
        return None
    vals = []
    for _ in range(samples):
        try:
            vals.append(int(open(f[0]).read().strip()))
        except (OSError, ValueError):
            return None
        time.sleep(period)
    return max(vals)


def time_passes(run, stream, nsets, passes=3, min_pass_s=0.1, max_launches=2000, warmup=None):
    """Warm up (50 launches, 500 for kernels under 0.5 ms), then `passes`
    passes of n back-to-back launches cycling over the input sets, each pass
    timed with a pair of HIP events on the launch stream; n is chosen so a
    pass lasts >= min_pass_s.  Returns (ms per launch of each pass, n)."""
    import torch
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # estimate
    for i in range(3):
        run(i)
    torch.cuda.synchronize()
    ev0.record(stream)
    for i in range(10):
        run(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    est = ev0.elapsed_time(ev1) / 10.0
    w = warmup if warmup is not None else (500 if est < 0.5 else 50)
    for i in range(w):
        run(i)
    n = int(min(max_launches, max(20, -(-min_pass_s * 1e3 // est))))
    n = max(n, nsets)
    out = []
    for _ in range(passes):
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(n):
            run(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        out.append(ev0.elapsed_time(ev1) / n)
    return out, n


def pass_stats(ms, flops, peak):
    med = float(np.median(ms))
    return {"ms_median": round(med, 6), "ms_min": round(float(min(ms)), 6), "ms_max": round(float(max(ms)), 6),
            "spread": round((max(ms) - min(ms)) / med, 4), "rate": round(flops / (med * 1e-3) / 1e12, 3),
            "rate_best": round(flops / (min(ms) * 1e-3) / 1e12, 3),
            "frac": round(flops / (med * 1e-3) / 1e12 / peak, 4)}


def sample_rows(M, n=16):
    """First two, last two (inside the partial tile when M is not a tile
    multiple) and evenly spaced rows between."""
    if M <= n:
        return np.arange(M)
    mid = np.linspace(2, M - 3, n - 4).round().astype(np.int64)
    return np.unique(np.concatenate([[0, 1], mid, [M - 2, M - 1]]))


def workload_label(d, prepacked=False):
    return (f"{d['name']} M={d['M']} N={d['N']} K={d['K']}" + (" bias" if d["bias"] is not None else "")
            + (" prepacked B" if prepacked else ""))


def bench_config(cfg, name, args, headline=None):
    """One workload of the suite: cold passes (with the clock sampled), hot
    passes, the prepacked-B call, and the output rows kept for the parity
    check (made later, in the CPU leg).  `headline` (a dict) receives the
    contract's K-step timing when this is the headline workload."""
    import torch
    from block_scaled_precision_02_amd import inputs
    import block_scaled_precision_02_amd as q

    log(f"[bench] config {cfg}: {name}")
    d0 = inputs.make(name)
    M, N, K = d0["M"], d0["N"], d0["K"]
    R = cold_sets(d0)
    flops = 2.0 * M * N * K
    peak = PEAK[dtype_of(d0)]
    sets = make_sets(d0, R)
    out = torch.empty((M, N + (-N) % 8), dtype=torch.bfloat16, device="cuda")[:, :N]
    stream = torch.cuda.current_stream()
    q.force_tile(-1)
    tile = q.select_tile({"i8": 0, "f8": 1, "e4m3": 2, "e2m1": 3}[dtype_of(d0)], M, N, K)
    rec = {"config": cfg, "workload": workload_label(d0), "dtype": dtype_of(d0), "unit": unit_of(d0),
           "peak": peak, "tile_id": tile, "input_sha256": inputs.digest(d0)[:16],
           "rotating_sets": R, "rotating_bytes": R * operand_bytes(d0)}
    run = Launcher(d0, sets, out, stream.cuda_stream)
    rec["gpu_busy_before"] = gpu_busy_percent()
    if headline is not None:
        # the contract's timing: W warmup steps, exactly K steps between two
        # synchronisations, HIP events on the launch stream for the kernel
        log(f"[bench] headline: warmup {args.warmup}, timing {args.steps} steps")
        for i in range(args.warmup):
            run(i)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for i in range(args.steps):
            run(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        headline.update(d=d0, wall=wall, kernel_ms=ev0.elapsed_time(ev1) / args.steps, tile=tile, R=R)
    with ClockSampler() as clk:
        ms, n = time_passes(run, stream, R)
    rec.update({"launches_per_pass": n, "passes": len(ms)})
    rec.update(pass_stats(ms, flops, peak))
    rec["algorithmic_bytes"] = min_bytes(d0)
    rec["traffic"] = traffic_bytes(name)
    sclk = clk.summary()
    rec["sclk_mhz"] = sclk
    if sclk is not None:
        rec["frac_at_sclk"] = round(rec["frac"] * 2400.0 / sclk["median"], 4)
    # parity rows of the last cold launch (every set holds the same values)
    rows = np.arange(M) if name in LATENCY_BOUND else sample_rows(M)
    torch.cuda.synchronize()
    got = out[torch.from_numpy(rows).cuda()].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    rec["_parity"] = [(d0, rows, got)]
    # hot: one input set, everything it can keep in the caches
    hot = Launcher(d0, sets[:1], out, stream.cuda_stream)
    hms, hn = time_passes(hot, stream, 1)
    rec["hot"] = dict(rotating_sets=1, launches_per_pass=hn, **pass_stats(hms, flops, peak))
    if name in LATENCY_BOUND:
        # the no-bias variant (its signed zeros checked by the parity leg),
        # and the host-side cost apart: calls replayed from one HIP graph
        d1 = dict(d0, bias=None)
        nb = make_sets(d1, 1)
        out1 = torch.empty_like(out)
        Launcher(d1, nb, out1, stream.cuda_stream)(0)
        torch.cuda.synchronize()
        got1 = out1.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        rec["_parity"].append((d1, np.arange(M), got1))
        ga = argparse.Namespace(graph=100, steps=1000, prepacked=False)
        rec["graph"] = time_graph(d0, sets, out, ga)
    else:
        pk = Launcher(d0, sets, out, stream.cuda_stream, prepacked=True)
        pms, pn = time_passes(pk, stream, R)
        rec["prepacked"] = dict(launches_per_pass=pn, **pass_stats(pms, flops, peak))
        ref = PAGES_REF_PREPACKED.get((name, M, N, K))
        if ref is not None:
            rec["prepacked"]["vs_pages"] = round(rec["prepacked"]["rate"] / ref, 4)
    ref = PAGES_REF.get((name, M, N, K))
    if ref is not None:
        rec["vs_pages"] = round(rec["rate"] / ref, 4)
    if (name, M, N, K) in PAGES_CONTEXT:
        rec["pages_context"] = PAGES_CONTEXT[(name, M, N, K)]
    del run, hot, sets, out
    torch.cuda.empty_cache()
    return rec


def parity_verdict(items):
    """The oracle on the kept output rows (CPU leg): INT8 bit for bit, FP8 /
    MX within the per-element bound and the cosine floor."""
    from tests import parity
    res = {"rows": 0, "pass": True}
    worst, cos = 0.0, 1.0
    for d, rows, got in items:
        ref, absdot, _ = parity.oracle_run(d, rows=rows)
        res["rows"] += len(rows)
        try:
            w, c = parity.compare(d, got, ref, absdot, d["name"])
            worst, cos = max(worst, w), min(cos, c)
        except AssertionError as e:
            res["pass"] = False
            res["error"] = str(e)[:300]
    if items[0][0]["kind"] == "i8":
        res["check"] = "bit-exact"
    else:
        res.update(check="|err| <= 1e-2*sum|ab| + 1 ulp, cos >= 0.99999", worst_err_over_bound=round(worst, 4),
                   cos=round(cos, 9))
    return res


def host_info():
    info = {"nproc": os.cpu_count()}
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            k, _, v = line.partition(":")
            if k.strip() == "Model name":
                info["model"] = v.strip()
            elif k.strip() == "Socket(s)":
                info["sockets"] = v.strip()
    except Exception:
        pass
    return info


def roofline_of(d, kernel_ms, name, shape=False, prepacked=False):
    M, N, K = d["M"], d["N"], d["K"]
    flops = 2.0 * M * N * K
    peak = PEAK[dtype_of(d)]
    nbytes = min_bytes(d)
    # below the ridge (peak ops per HBM byte) the call is bound by HBM, not MFMA
    if flops / nbytes < peak * 1e12 / (HBM_GBPS * 1e9):
        gbps = nbytes / (kernel_ms * 1e-3) / 1e9
        r = {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_GBPS, "unit": "GB/s",
             "frac": round(gbps / HBM_GBPS, 4)}
    else:
        achieved = flops / (kernel_ms * 1e-3) / 1e12
        r = {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": unit_of(d),
             "frac": round(achieved / peak, 4)}
    r.update({"traffic": None if (shape or prepacked) else traffic_bytes(name), "kernel_ms": round(kernel_ms, 6),
              "algorithmic_bytes": nbytes})
    return r


DTYPE_NAME = {"i8": "int8", "f8": "e4m3", "f8b": "e4m3", "e4m3": "mxfp8-e4m3", "e2m1": "mxfp4-e2m1",
              "e4m3/e2m1": "mx-e4m3xe2m1", "e2m1/e4m3": "mx-e2m1xe4m3", "e2m3": "mxfp6-e2m3",
              "e3m2": "mxfp6-e3m2"}


def suite(args):
    """The default run: the headline plus every workload's per-config record."""
    import torch
    headline = {}
    recs = []
    for cfg, name in SUITE:
        if args.no_suite and name != HEADLINE:
            continue
        recs.append(bench_config(cfg, name, args, headline if name == HEADLINE else None))
    d = headline["d"]
    M, N, K = d["M"], d["N"], d["K"]
    ms_per_step = headline["wall"] * 1e3 / args.steps
    flops = 2.0 * M * N * K
    value = flops / (ms_per_step * 1e-3) / 1e12
    peak = PEAK[dtype_of(d)]
    res = {
        "metric": METRIC, "value": round(value, 3), "unit": unit_of(d), "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": DTYPE_NAME[dtype_of(d)], "data": "synthetic",
        "config": {"workload": workload_label(d), "tile_id": headline["tile"], "rotating_sets": headline["R"],
                   "pct_of_peak": round(100 * value / peak, 2)},
        "roofline": roofline_of(d, headline["kernel_ms"], HEADLINE),
        "cpu_baseline": None,
    }
    if (HEADLINE, M, N, K) in PAGES_CONTEXT:
        res["config"]["pages_context"] = PAGES_CONTEXT[(HEADLINE, M, N, K)]
    torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        log("[bench] cpu leg: oracle baseline and parity of the kept rows")
        res["cpu_baseline"] = cpu_baseline(d, args.cpu_seconds)
        for r in recs:
            log(f"[bench] parity config {r['config']}")
            r["parity"] = parity_verdict(r["_parity"])
    for r in recs:
        del r["_parity"]
    res["per_config"] = recs
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None,
                    help="time one workload (default: the headline and every workload's per-config record)")
    ap.add_argument("--no-suite", action="store_true", help="default run: the headline only")
    ap.add_argument("--rot", type=int, default=None, help="rotating input sets")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tile", type=int, default=-1, help="force a tile id (-1: the table's choice)")
    ap.add_argument("--shape", default=None, metavar="M,N,K",
                    help="run the workload's recipe at another shape (e.g. the skinny-M cases)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="instead: time a plain device copy of this many bytes (the "
                         "reference kernel for scaling FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--prepacked", action="store_true",
                    help="B prepacked once (qgemm_prepack_b) and the _prepacked entry points timed")
    ap.add_argument("--quant", default=None, choices=["f8", "mxfp8", "mxfp4", "f8_block"],
                    help="instead: time the activation quantiser on the A shape of that workload")
    ap.add_argument("--graph", type=int, default=0, metavar="N",
                    help="also time N calls captured in one HIP graph and replayed (the host-side checks and the "
                         "per-call launch overhead apart); the replays' output is checked against the eager call's")
    ap.add_argument("--traffic-from", default=None, metavar="DIR",
                    help="instead: write profiles/traffic.json from the rocprofv3 FETCH_SIZE / "
                         "WRITE_SIZE runs under DIR (no GPU needed)")
    args = ap.parse_args()
    if args.traffic_from:
        print(json.dumps(write_traffic(args.traffic_from, TRAFFIC_WORKLOADS)))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this GEMM library has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from block_scaled_precision_02_amd import inputs
    import block_scaled_precision_02_amd as q

    torch.cuda.set_device(0)
    if args.copy_bytes:
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_bytes, "launches": args.steps}), flush=True)
        return
    if args.quant:
        print(json.dumps(bench_quant(args)), flush=True)
        return
    if args.workload is None and not (args.shape or args.prepacked or args.graph or args.tile >= 0 or args.rot):
        print(json.dumps(suite(args)), flush=True)
        return
    name = args.workload or HEADLINE
    shape = {}
    if args.shape:
        shape = dict(zip("MNK", (int(v) for v in args.shape.split(","))))
    d0 = inputs.make(name, **shape)
    R = args.rot or cold_sets(d0)
    log(f"[bench] {name} {shape or ''} x{R}")
    sets = make_sets(d0, R)
    M, N, K = d0["M"], d0["N"], d0["K"]
    out = torch.empty((M, N + (-N) % 8), dtype=torch.bfloat16, device="cuda")[:, :N]
    stream = torch.cuda.current_stream()
    run = Launcher(d0, sets, out, stream.cuda_stream, prepacked=args.prepacked)
    tile = q.select_tile({"i8": 0, "f8": 1, "e4m3": 2, "e2m1": 3, "f8b": 4, "e4m3/e2m1": 5, "e2m3": 6,
                          "e3m2": 7, "e2m1/e4m3": 8}[dtype_of(d0)], M, N, K)
    if args.tile >= 0:
        q.force_tile(args.tile)
        tile = args.tile

    log(f"[bench] warmup {args.warmup}")
    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    with ClockSampler() as clk:
        t0 = time.perf_counter()
        ev0.record(stream)
        for i in range(args.steps):
            run(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    kernel_ms = ev0.elapsed_time(ev1) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    flops = 2.0 * M * N * K
    value = flops / (ms_per_step * 1e-3) / 1e12
    peak = PEAK[dtype_of(d0)]
    ref = (PAGES_REF_PREPACKED if args.prepacked else PAGES_REF).get((name, M, N, K))
    res = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": unit_of(d0),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / ref, 4) if ref else None,
        "dtype": DTYPE_NAME[dtype_of(d0)],
        "data": "synthetic",
        "config": {"workload": workload_label(d0, args.prepacked), "tile_id": tile, "rotating_sets": R,
                   "pct_of_peak": round(100 * value / peak, 2), "sclk_mhz": clk.summary()},
        "roofline": roofline_of(d0, kernel_ms, name, bool(shape), args.prepacked),
        "cpu_baseline": None,
    }
    if (name, M, N, K) in PAGES_CONTEXT:
        res["config"]["pages_context"] = PAGES_CONTEXT[(name, M, N, K)]
    if args.graph:
        res["config"]["graph"] = time_graph(d0, sets, out, args)
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(d0, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
