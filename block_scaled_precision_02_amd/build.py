"""Build libqgemm.so in-tree: hipcc, gfx950 only.

    python -m block_scaled_precision_02_amd.build              # build libqgemm.so (+ the sync twin)
    python -m block_scaled_precision_02_amd.build --resources  # per-kernel register / LDS audit

Every HIP source under csrc/ compiles to an object in parallel, then one
shared library is linked next to this file.  Flags: -O3, no fast-math, no
floating-point contraction (the epilogue's multiply-then-add order is part of
the result), and packed-FP32 instructions disabled.
"""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqgemm.so")
SOURCES = ["qgemm_api.cpp", "qgemm_i8.hip", "qgemm_f8.hip", "qgemm_mx8.hip", "qgemm_mx4.hip", "qgemm_f8b.hip", "qgemm_mx84.hip", "qgemm_mx48.hip", "qgemm_mx4h.hip", "qgemm_mx6.hip",
           "qgemm_quant.hip", "qgemm_pack.hip"]
# Per-source extra flags.  The blockscale kernel folds its MFMA partial sums
# into the totals with VALU FMAs every 128 K elements; keeping the MFMA
# results in VGPRs (rather than the accumulator registers, which the VALU
# reaches only through a v_accvgpr_read per value) halves that VALU work.
EXTRA_FLAGS = {"qgemm_f8b.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-fno-fast-math", "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


# The conservative-sync twin (test infrastructure): the same sources with
# QGEMM_SYNC_TWIN=1, which drains every wait and adds a barrier at every stage
# boundary of the LDS-staged kernels; its outputs must equal the library's bit
# for bit.
BUILD_SYNC = os.path.join(HERE, "_build_sync")
LIB_SYNC = os.path.join(HERE, "libqgemm_sync.so")


def _compile(src, twin=False):
    obj = os.path.join(BUILD_SYNC if twin else BUILD, src + ".o")
    cmd = ([HIPCC] + FLAGS + EXTRA_FLAGS.get(src, []) + (["-DQGEMM_SYNC_TWIN=1"] if twin else []) +
           ["-c", os.path.join(CSRC, src), "-o", obj])
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, lib)


def build(jobs=None, twin=True):
    """Build libqgemm.so and (twin=True) the conservative-sync twin
    libqgemm_sync.so, every object compiled in one parallel pass."""
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(BUILD_SYNC, exist_ok=True)
    work = [(src, False) for src in SOURCES] + ([(src, True) for src in SOURCES] if twin else [])
    jobs = jobs or min(len(work), 2 * (os.cpu_count() or 4), 16)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda w: _compile(*w), work))
    _link(objs[:len(SOURCES)], LIB)
    if twin:
        _link(objs[len(SOURCES):], LIB_SYNC)
    return LIB


# ------------------------------------------------------------ resource audit

_REMARKS = (("VGPRs", "VGPRs"), ("AGPRs", "AGPRs"), ("TotalSGPRs", "SGPRs"), ("ScratchSize [bytes/lane]", "scratch B/lane"),
            ("VGPRs Spill", "VGPR spill"), ("SGPRs Spill", "SGPR spill"), ("LDS Size [bytes/block]", "LDS B"),
            ("Occupancy [waves/SIMD]", "waves/SIMD"))


def _audit(src):
    import re
    cmd = ([HIPCC] + FLAGS + EXTRA_FLAGS.get(src, []) + ["-Rpass-analysis=kernel-resource-usage", "-c",
           os.path.join(CSRC, src), "-o", os.path.join(BUILD, src + ".audit.o")])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}")
    rows, kern, vals = [], None, {}
    for line in r.stderr.splitlines():
        m = re.search(r"remark:\s+(.*?):\s+(\S+)\s+\[-Rpass-analysis", line)
        if not m:
            continue
        key, val = m.group(1).strip(), m.group(2)
        if key == "Function Name":
            if kern:
                rows.append((kern, vals))
            kern, vals = val, {}
        else:
            vals[key] = val
    if kern:
        rows.append((kern, vals))
    return src, rows


def resources(out=sys.stdout):
    """Compile every HIP source with the compiler's per-kernel resource
    remarks and print one markdown row per kernel instantiation."""
    import shutil
    os.makedirs(BUILD, exist_ok=True)
    filt = shutil.which("llvm-cxxfilt") or shutil.which("c++filt")
    srcs = [s for s in SOURCES if s.endswith(".hip")]
    with concurrent.futures.ThreadPoolExecutor(min(len(srcs), os.cpu_count() or 4, 16)) as ex:
        results = list(ex.map(_audit, srcs))
    print("| Source | Kernel | " + " | ".join(h for _, h in _REMARKS) + " |", file=out)
    print("|---|---|" + "---|" * len(_REMARKS), file=out)
    for src, rows in results:
        names = [k for k, _ in rows]
        if filt and names:
            dem = subprocess.run([filt], input="\n".join(names), capture_output=True, text=True).stdout.splitlines()
            if len(dem) == len(names):
                names = dem
        for name, (_, vals) in zip(names, rows):
            name = name.replace("(qgemm::Params)", "").replace("void qgemm::", "").strip()
            print(f"| {src} | `{name}` | " + " | ".join(vals.get(k, "-") for k, _ in _REMARKS) + " |", file=out)


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "--resources":
        resources()
        sys.exit(0)
    print(build(twin="--no-twin" not in sys.argv))
    sys.exit(0)
