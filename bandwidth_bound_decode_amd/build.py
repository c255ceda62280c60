"""Build libbbd_gemv.so in-tree: hipcc for the gfx950 kernels, g++ for the host-only plan.

Every HIP translation unit is compiled with packed-fp32 instructions disabled
(-target-feature -packed-fp32-ops); the kernels need none and the flag keeps the compiler
from forming them out of scalar float code.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libbbd_gemv.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-Werror",
             f"-I{INCLUDE}", f"-I{CSRC}"]


RESOURCE_REPORT = os.path.join(LIB_DIR, "kernel_resources.json")
HIP_UNITS = ("gemv", "whole", "batch", "mfma", "int4", "norm", "chain", "calib")
REMARK = "[-Rpass-analysis=kernel-resource-usage]"


def _run(cmd):
    proc = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    lines = [l for l in proc.stderr.splitlines() if noise not in l]
    remarks = [l for l in lines if REMARK in l]
    # drop the remarks and the source excerpts the compiler prints under each of them
    err = "\n".join(l for l in lines if REMARK not in l and "remark:" not in l
                    and not re.match(r"^\s*(\d+\s*)?[|^]", l))
    if proc.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return remarks


def _resources(remarks):
    """Per-kernel resource usage from the compiler's kernel-resource-usage remarks."""
    kernels, cur = {}, None
    for line in remarks:
        body = line.split("remark:", 1)[1].replace(REMARK, "").strip()
        key, _, val = body.partition(":")
        key, val = key.strip(), val.strip()
        if key == "Function Name":
            cur = kernels.setdefault(val, {})
        elif cur is not None:
            cur[key] = val
    return kernels


def _check_resources(kernels):
    """Refuse a library in which any kernel uses scratch memory or spills VGPRs. (SGPR spills
    land in VGPR lanes, not memory; they are recorded in the report but allowed.)"""
    if not kernels:
        raise RuntimeError("the compiler reported no kernel resource usage")
    bad = [name for name, r in kernels.items()
           if r.get("ScratchSize [bytes/lane]", "0") != "0" or r.get("VGPRs Spill", "0") != "0"]
    if bad:
        raise RuntimeError(f"kernels using scratch memory or spilling VGPRs: {bad[:5]}")


def build(out: str = LIB_PATH, save_temps: str | None = None) -> str:
    """Compile the library into `out` (default: the package's lib/ directory)."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    with tempfile.TemporaryDirectory() as tmp:
        plan_o = os.path.join(tmp, "plan.o")
        _run(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, "plan.cpp"), "-o", plan_o])
        objs, remarks = [plan_o], []

        def compile_unit(unit):
            obj = os.path.join(tmp, unit + ".o")
            rem = _run([HIPCC, *HIP_FLAGS, "-Rpass-analysis=kernel-resource-usage",
                        "-c", os.path.join(CSRC, unit + ".hip"), "-o", obj])
            if save_temps:
                # the device assembly, for reading the generated code
                os.makedirs(save_temps, exist_ok=True)
                _run([HIPCC, *HIP_FLAGS, "--cuda-device-only", "-S",
                      os.path.join(CSRC, unit + ".hip"),
                      "-o", os.path.join(save_temps, f"{unit}-hip-amdgcn-amd-amdhsa-gfx950.s")])
            return obj, rem

        # one compiler process per translation unit, at most as many as the host's CPUs
        workers = max(1, min(len(HIP_UNITS), len(os.sched_getaffinity(0)), 16))
        with ThreadPoolExecutor(max_workers=workers) as pool:
            for obj, rem in pool.map(compile_unit, HIP_UNITS):
                objs.append(obj)
                remarks += rem
        tmp_out = out + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_out])
        kernels = _resources(remarks)
        _check_resources(kernels)
        os.replace(tmp_out, out)
    if out == LIB_PATH:
        import json
        with open(RESOURCE_REPORT, "w") as f:
            json.dump(kernels, f, indent=1, sort_keys=True)
    return out


if __name__ == "__main__":
    print(build())
