"""Build liblmtopk.so in-tree for gfx950.

    python lm_head_projection_amd/build.py        # or lm_head_projection_amd.build.build()

The HIP translation units (kernels + launchers, one per path) are compiled
by hipcc for gfx950 in parallel; the C ABI layer is plain host C++ compiled
by g++; hipcc links them all into lm_head_projection_amd/_lib/liblmtopk.so.
The benchmark's read-rate probe (csrc/probe_read.hip) is built beside it as
_lib/libprobe_read.so.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(PKG, "_lib")
LIB = os.path.join(OUT_DIR, "liblmtopk.so")
PROBE_LIB = os.path.join(OUT_DIR, "libprobe_read.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_SOURCES = ["lmtopk_binary.hip", "lmtopk_dense.hip", "lmtopk_select_merge.hip",
               "lmtopk_noalloc.hip"]
# Packed-fp32 instructions stay off in every device compile.
DEVICE_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-pass-failed",
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
    cmds, objs = [], []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        cmds.append([HIPCC, *DEVICE_FLAGS, *inc, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    a_obj = os.path.join(BUILD_DIR, "lmtopk_api.o")
    cxx = shutil.which("g++") or "g++"
    cmds.append([cxx, *HOST_FLAGS, *inc, "-c", os.path.join(CSRC, "lmtopk_api.cpp"), "-o", a_obj])
    objs.append(a_obj)
    with ThreadPoolExecutor(max_workers=len(cmds)) as pool:
        for f in [pool.submit(_run, c, verbose) for c in cmds]:
            f.result()
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    # the benchmark's read-rate probe: a library of its own, not liblmtopk
    tmp = PROBE_LIB + ".tmp"
    _run([HIPCC, *DEVICE_FLAGS, "-shared", os.path.join(CSRC, "probe_read.hip"), "-o", tmp], verbose)
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
