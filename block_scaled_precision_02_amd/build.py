"""Build libqgemm.so in-tree: hipcc, gfx950 only.

    python -m block_scaled_precision_02_amd.build

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
SOURCES = ["qgemm_api.cpp", "qgemm_i8.hip", "qgemm_f8.hip", "qgemm_mx8.hip", "qgemm_mx4.hip", "qgemm_f8b.hip", "qgemm_mx84.hip",
           "qgemm_quant.hip", "qgemm_pack.hip"]
# Per-source extra flags.  The blockscale kernel folds its MFMA partial sums
# into the totals with VALU FMAs every 128 K elements; keeping the MFMA
# results in VGPRs (rather than the accumulator registers, which the VALU
# reaches only through a v_accvgpr_read per value) halves that VALU work.
EXTRA_FLAGS = {"qgemm_f8b.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-fno-fast-math", "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src):
    obj = os.path.join(BUILD, src + ".o")
    cmd = [HIPCC] + FLAGS + EXTRA_FLAGS.get(src, []) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return obj


def build(jobs=None):
    os.makedirs(BUILD, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 4, 16)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
    sys.exit(0)
