"""The C ABI's host layer under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

lmtopk_api.cpp (argument checks, geometry, merge plan) is compiled once more
by g++ with -fsanitize=address,undefined (host code only; the HIP objects of
the regular build are linked unchanged), and tests/test_abi.py runs against
that library in a child process with the ASan runtime preloaded and every
UBSan report fatal.  A read past a buffer, a signed overflow in the size
arithmetic or a misaligned access in the host layer then fails the run."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "_build")
OUT = os.path.join(BUILD, "sanitized")
HIP_OBJECTS = ["lmtopk_binary.o", "lmtopk_dense.o", "lmtopk_select_merge.o", "lmtopk_noalloc.o"]


def _libasan():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_abi_under_asan_and_ubsan():
    objs = [os.path.join(BUILD, o) for o in HIP_OBJECTS]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("the regular build's objects are missing (run the build first)")
    asan = _libasan()
    if asan is None:
        pytest.skip("no libasan for this g++")
    os.makedirs(OUT, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "lm_head_projection_amd", "csrc")]
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
    api_o = os.path.join(OUT, "lmtopk_api.o")
    lib = os.path.join(OUT, "liblmtopk.so")
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-fPIC", *san, *inc, "-c",
                    os.path.join(ROOT, "lm_head_projection_amd", "csrc", "lmtopk_api.cpp"), "-o", api_o],
                   check=True)
    subprocess.run(["g++", "-shared", *san, api_o, *objs, "-L/opt/rocm/lib", "-lamdhip64",
                    "-Wl,-rpath,/opt/rocm/lib", "-o", lib], check=True)
    env = dict(os.environ, LD_PRELOAD=asan, LMTOPK_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "passed" in r.stdout
