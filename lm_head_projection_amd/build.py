"""Build liblmtopk.so in-tree for gfx950.

    python -m lm_head_projection_amd.build        # or lm_head_projection_amd.build.build()

The HIP translation unit (kernels + launchers) is compiled by hipcc for
gfx950; the C ABI layer is plain host C++ compiled by g++; hipcc links both
into lm_head_projection_amd/_lib/liblmtopk.so.
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(OUT_DIR, "liblmtopk.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed-fp32 instructions stay off in every device compile.
DEVICE_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd[:2])} ... (exit {r.returncode})")
    if verbose and (r.stdout or r.stderr):
        sys.stderr.write(r.stdout + r.stderr)


def build(verbose=False):
    os.makedirs(OUT_DIR, exist_ok=True)
    os.makedirs(BUILD_DIR, exist_ok=True)
    inc = ["-I", INCLUDE, "-I", CSRC]
    k_obj = os.path.join(BUILD_DIR, "lmtopk_kernels.o")
    a_obj = os.path.join(BUILD_DIR, "lmtopk_api.o")
    _run([HIPCC, *DEVICE_FLAGS, *inc, "-c", os.path.join(CSRC, "lmtopk_kernels.hip"), "-o", k_obj],
         verbose)
    cxx = shutil.which("g++") or "g++"
    _run([cxx, *HOST_FLAGS, *inc, "-c", os.path.join(CSRC, "lmtopk_api.cpp"), "-o", a_obj], verbose)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", k_obj, a_obj, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
