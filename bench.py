"""Benchmark of the scaled low-precision GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one call of the GEMM (argument checks, tile choice, one kernel:
tile schedule, HBM->LDS staging, MFMA K loop, fused scale/bias epilogue) on
one batch of seeded synthetic inputs already resident in HBM.  The default
workload is the INT8 rowwise projection M=30000 N=21504 K=5376 with bias;
--workload picks another (i8_small, f8_ptpc, mxfp8, mxfp4, i8_qkv, and
f8_block: FP8 with fp32 scales per 128-element K block, 16384x7168x2048;
mx_a8w4: MX e4m3 A x e2m1 B, 8192^3).

Prints one JSON line: effective TOPS/TFLOPS = 2MNK / t, the roofline of the
kernel (achieved over the dense MFMA peak of its dtype, from HIP events on
the launch stream), and the CPU oracle timed on a bounded sample of the same
workload on this host.
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
# (e4m3 x e2m1 MX runs at the e4m3 rate: the scaled MFMA takes 64 cycles when
# either operand is 8-bit)
PEAK = {"i8": 5000.0, "f8": 5000.0, "f8b": 5000.0, "e4m3": 5000.0, "e2m1": 10100.0, "e4m3/e2m1": 5000.0}
HBM_GBPS = 8000.0
# The pages' numbers for exactly these workloads (2MNK / their time where they
# give a time), quoted by vs_baseline; context, not targets:
#  - INT8 30000x21504x5376: 209.9 TOPS on an RX 9070 XT (comfy-kitchen PR #174,
#    Performance) -- another GPU;
#  - MXFP8 16384x7168x2048: 246.2 us and 32768x7168x1792: 462.2 us, FP8
#    blockscale 16384x7168x2048: 362.3 us, all on MI355X (ROCm/mori PR #806,
#    commit message table; its MXFP8 reads a packed scale layout);
#  - MXFP4 8192^3: 5034 TFLOPS on MI355X (ROCm/FlyDSL PR #990, Performance).
PAGES_REF = {
    ("i8_qkv", 30000, 21504, 5376): 209.9,
    ("mxfp8", 16384, 7168, 2048): 2.0 * 16384 * 7168 * 2048 / 246.2e-6 / 1e12,
    ("mxfp8", 32768, 7168, 1792): 2.0 * 32768 * 7168 * 1792 / 462.2e-6 / 1e12,
    ("f8_block", 16384, 7168, 2048): 2.0 * 16384 * 7168 * 2048 / 362.3e-6 / 1e12,
    ("mxfp4", 8192, 8192, 8192): 5034.0,
}
# Rotating input sets so operands are not served from the 256 MB MALL.
ROT = {"i8_small": 1, "f8_ptpc": 8, "mxfp8": 2, "mxfp4": 3, "i8_qkv": 2, "f8_block": 2, "mx_a8w4": 3}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def dtype_of(d):
    return d["kind"] if d["kind"] != "mx" else d["fmt"]


def unit_of(d):
    return "TOPS" if d["kind"] == "i8" else "TFLOPS"


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
                pb = q.qgemm_prepack_b32(s["B"]).data
                s["Bp"] = pb
                a = (0, 1, s["A"].data_ptr(), s["A"].stride(0), pb.data_ptr(), s["scale_a"].data_ptr(),
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
                    fmt = 0 if d["fmt"] == "e4m3" else 1
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
                fmt = 0 if d["fmt"] == "e4m3" else 1
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
    ab = M * (K // 2 if fa == "e2m1" else K) + N * (K // 2 if fb == "e2m1" else K)
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
    first to calibrate, then enough rows for about target_s seconds."""
    import oracle
    from tests import parity
    rows = np.arange(min(2, d["M"]))
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
            "kind": "oracle",
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="i8_qkv")
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
        print(json.dumps(write_traffic(args.traffic_from, ["i8_qkv", "mxfp4", "f8_block", "mx_a8w4"])))
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
    name = args.workload
    shape = {}
    if args.shape:
        shape = dict(zip("MNK", (int(v) for v in args.shape.split(","))))
    R = args.rot or ROT[name]
    log(f"[bench] generating {name} {shape or ''} x{R}")
    d0 = inputs.make(name, **shape)
    sets = [upload(d0)]
    for r in range(1, R):
        sets.append(upload(inputs.make(name, rot=r, **shape)))
    M, N, K = d0["M"], d0["N"], d0["K"]
    out = torch.empty((M, N + (-N) % 8), dtype=torch.bfloat16, device="cuda")[:, :N]
    stream = torch.cuda.current_stream()
    run = Launcher(d0, sets, out, stream.cuda_stream, prepacked=args.prepacked)
    tile = q.select_tile({"i8": 0, "f8": 1, "e4m3": 2, "e2m1": 3, "f8b": 4, "e4m3/e2m1": 5}[dtype_of(d0)], M, N, K)
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
    achieved = flops / (kernel_ms * 1e-3) / 1e12
    peak = PEAK[dtype_of(d0)]
    nbytes = min_bytes(d0)
    # below the ridge (peak ops per HBM byte) the call is bound by HBM, not MFMA
    hbm_bound = flops / nbytes < peak * 1e12 / (HBM_GBPS * 1e9)
    if hbm_bound:
        gbps = nbytes / (kernel_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_GBPS, "unit": "GB/s",
                    "frac": round(gbps / HBM_GBPS, 4)}
    else:
        roofline = {"bound": "mfma", "achieved": round(achieved, 3), "peak": peak, "unit": unit_of(d0),
                    "frac": round(achieved / peak, 4)}
    roofline.update({"traffic": None if (shape or args.prepacked) else traffic_bytes(name),
                     "kernel_ms": round(kernel_ms, 6),
                     "algorithmic_bytes": nbytes})

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
        "vs_baseline": round(value / PAGES_REF[(name, M, N, K)], 4) if (name, M, N, K) in PAGES_REF else None,
        "dtype": {"i8": "int8", "f8": "e4m3", "f8b": "e4m3", "e4m3": "mxfp8-e4m3",
                  "e2m1": "mxfp4-e2m1", "e4m3/e2m1": "mx-e4m3xe2m1"}[dtype_of(d0)],
        "data": "synthetic",
        "config": {"workload": f"{name} M={M} N={N} K={K}" + (" bias" if d0["bias"] is not None else "")
                   + (" prepacked B" if args.prepacked else ""),
                   "tile_id": tile, "rotating_sets": R, "pct_of_peak": round(100 * value / peak, 2)},
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if args.graph:
        res["config"]["graph"] = time_graph(d0, sets, out, args)
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(d0, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
