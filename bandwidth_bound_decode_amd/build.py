"""Build libbbd_gemv.so in-tree: hipcc for the gfx950 kernels, g++ for the host-only plan.

Every HIP translation unit is compiled with packed-fp32 instructions disabled
(-target-feature -packed-fp32-ops); the kernels need none and the flag keeps the compiler
from forming them out of scalar float code.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

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


def _run(cmd):
    proc = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in proc.stderr.splitlines() if noise not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")


def build(out: str = LIB_PATH, save_temps: str | None = None) -> str:
    """Compile the library into `out` (default: the package's lib/ directory)."""
    os.makedirs(os.path.dirname(out), exist_ok=True)
    with tempfile.TemporaryDirectory() as tmp:
        plan_o = os.path.join(tmp, "plan.o")
        gemv_o = os.path.join(tmp, "gemv.o")
        _run(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, "plan.cpp"), "-o", plan_o])
        extra = [f"-save-temps={save_temps}"] if save_temps else []
        cwd = os.getcwd()
        try:
            if save_temps:
                os.makedirs(save_temps, exist_ok=True)
                os.chdir(save_temps)
            _run([HIPCC, *HIP_FLAGS, *extra, "-c", os.path.join(CSRC, "gemv.hip"), "-o", gemv_o])
        finally:
            os.chdir(cwd)
        tmp_out = out + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", plan_o, gemv_o,
              "-o", tmp_out])
        os.replace(tmp_out, out)
    return out


if __name__ == "__main__":
    print(build())
