"""The kernel argument layout of the library's own gfx950 code objects (CPU
only: the code objects are read from the built libqgemm.so, nothing runs).

Every GEMM kernel takes one argument, the Params block, by value.  Some
LDS-fetch kernels read launch arguments a second time after their K loop,
through the kernarg segment pointer, as a Params at offset 0 of that
segment: the AMDGPU code-object ABI places the explicit arguments first.
This test checks that layout in the metadata the compiler wrote: each
qgemm kernel lists exactly one by-value argument, at offset 0, as large as
the whole explicit part of the segment."""
import os
import re
import shutil
import subprocess

import pytest
import yaml

import block_scaled_precision_02_amd as q

LLVM = "/opt/rocm/llvm/bin"


def _code_objects(tmp_path):
    lib = q.LIB_PATH
    if not os.path.exists(lib):
        pytest.skip("libqgemm.so is not built")
    for tool in ("llvm-objdump", "llvm-readelf"):
        if not os.path.exists(os.path.join(LLVM, tool)):
            pytest.skip(f"{tool} is not installed")
    # llvm-objdump --offloading writes the bundles next to its input: work on a copy
    copy = tmp_path / "libqgemm.so"
    shutil.copyfile(lib, copy)
    subprocess.run([os.path.join(LLVM, "llvm-objdump"), "--offloading", str(copy)], cwd=tmp_path,
                   check=True, capture_output=True)
    objs = sorted(p for p in tmp_path.iterdir() if "amdgcn-amd-amdhsa" in p.name and "gfx950" in p.name)
    assert objs, "no gfx950 code object in libqgemm.so"
    return objs


def _kernels(notes):
    """(name, [(offset, size, value_kind), ...], kernarg_segment_size) per
    kernel, from the code object's metadata note (a YAML document)."""
    text = notes.split("amdhsa.kernels:", 1)[1]
    end = re.search(r"^\s*\.\.\.\s*$", text, re.M)
    doc = yaml.safe_load("amdhsa.kernels:" + (text[:end.start()] if end else text))
    out = []
    for k in doc["amdhsa.kernels"]:
        args = [(a[".offset"], a[".size"], a[".value_kind"]) for a in k.get(".args", [])]
        out.append((k[".name"], args, k.get(".kernarg_segment_size")))
    return out


def test_params_is_the_only_argument_at_offset_zero(tmp_path):
    seen = 0
    for obj in _code_objects(tmp_path):
        notes = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", str(obj)], check=True,
                               capture_output=True, text=True).stdout
        if "amdhsa.kernels:" not in notes:
            continue
        for name, args, seg in _kernels(notes):
            if "qgemm" not in name or "Params" not in name:
                continue
            seen += 1
            explicit = [a for a in args if not a[2].startswith("hidden_")]
            assert len(explicit) == 1, f"{name}: explicit arguments {explicit}"
            off, size, kind = explicit[0]
            assert (off, kind) == (0, "by_value"), f"{name}: Params at offset {off} ({kind})"
            assert size >= 132 and size % 8 == 0, f"{name}: Params of {size} bytes"
            assert seg is not None and seg >= size, f"{name}: kernarg segment of {seg} bytes"
    assert seen >= 100, f"only {seen} qgemm kernels found in the code objects"
