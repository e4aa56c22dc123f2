"""The C ABI on the host (CPU only): the library loads, exports every function
include/lmtopk.h declares, and rejects every invalid argument with its status
code before any HIP call.  Pointer arguments here are small fabricated
integers that the library must never dereference."""

import ctypes
import os
import re
import shutil
import subprocess
import tempfile

import pytest

import lm_head_projection_amd as lt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lmtopk.h")

OK, NULL, SHAPE, K, GROUP, DTYPE, ALIGN, WORKSPACE, OPTIONS, HIP = range(10)
A = 4096      # a fabricated, 16-byte aligned "device pointer"
ODD = 4100    # a fabricated, misaligned one
BIG = 1 << 40


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lmtopk_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function():
    names = declared_functions()
    assert {"lmtopk_pack_binary", "lmtopk_binary", "lmtopk_dense", "lmtopk_select"} <= set(names)
    lib = ctypes.CDLL(lt.library_path())
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", lt.library_path()], capture_output=True,
                         text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}\b", out), f"{n} not exported"


def test_layout_and_sizes():
    assert lt.layout_version() == 1
    assert lt.packed_bytes(248320, 5120) == (158924800, 39731200)   # signs + fp32 scales
    assert lt.packed_bytes(32001, 2048) == (32064 * 2048 // 8, 32064 * 16 * 4)
    assert lt.packed_bytes(1, 640) == (64 * 640 // 8, 64 * 8 * 4)   # G=5 pads to 8 scales
    # completion counter (256 B) + chunk heads (243 x 4 x 8 B rounded to 256) + chunk
    # the completion counter (256 B) and eight key histograms (8 x 2,048 x 4
    # B), then the heads and candidates of the flagship (243 chunks x 50 x 8 B
    # rounded to 256) + log-sum-exp pairs (243 chunks x 8 B, rounded to 256);
    # one workgroup merges them, no second region
    sync = 256 + 8 * 2048 * 4
    assert lt.workspace_bytes(1, 248320, 50) == sync + 7936 + 97280 + 2048
    # k >= chunk rows: every chunk offers all its rows, and the merge needs two
    # levels (the first level's 16 segments per row also post their counts)
    assert lt.workspace_bytes(8, 248320, 1024) == (sync + 8 * 243 * 32 + 8 * 243 * 1024 * 8
                                                   + 8 * 16 * 1024 * 8 + 15616 + 512)


def test_workspace_covers_the_two_wave_plan():
    # V = 128,256: 126 chunks of 1,024 rows would leave half of the CUs idle,
    # so the binary path scores 251 chunks of 512 rows with two waves per tile
    # (16 waves per chunk); the size query covers that plan as well as the
    # other paths' 126 chunks
    sync = 256 + 8 * 2048 * 4                 # completion counter, key histograms
    split = sync + 8192 + 100608 + 2048      # 251 x 4 x 8 -> 8,192; 251 x 50 x 8 -> 100,608;
    plain = sync + 4096 + 50432 + 1024       # 251 x 8 -> 2,048 (vs 126 chunks)
    assert lt.workspace_bytes(1, 128256, 50) == max(split, plain) == split
    kw = dict(V=128256, H=4096, k=50)
    assert _binary(**kw, ws_bytes=split - 1) == WORKSPACE
    assert _binary(**kw, ws_bytes=split) == HIP  # every host check passed; no device here
    assert _dense(**kw, M=1, ws_bytes=plain - 1) == WORKSPACE
    assert _dense(**kw, M=1, ws_bytes=plain) == HIP
    # the plan the binary path reports: 251 chunks of 512 rows, 16 waves each;
    # explicit sizes up to 512 rows take two waves per tile as well
    assert lt.binary_plan(1, 128256, 4096, 50) == (512, 251, 16)
    assert lt.binary_plan(1, 128256, 4096, 50, chunk_rows=256) == (256, 501, 8)
    assert lt.binary_plan(1, 128256, 4096, 50, chunk_rows=1024) == (1024, 126, 16)
    assert lt.binary_plan(1, 248320, 5120, 50) == (1024, 243, 16)
    assert lt.binary_plan(2, 248320, 5120, 50, chunk_rows=2048) == (2048, 122, 8)
    assert lt.binary_plan(1, 40, 128, 40) == (64, 1, 2)
    # the largest activation block (M * H = 65,536) still fits the exchange area
    assert lt.binary_plan(8, 5000, 8192, 50) == (512, 10, 16)
    # k above the fused merge's range keeps 1,024-row chunks (the merge is a
    # separate launch either way)
    assert lt.binary_plan(1, 128256, 4096, 300) == (1024, 126, 16)
    lib = lt._lib
    c = ctypes.c_int32()
    assert lib.lmtopk_binary_plan(1, 1000, 200, 5, None, ctypes.byref(c), ctypes.byref(c),
                                  ctypes.byref(c)) == GROUP
    assert lib.lmtopk_binary_plan(1, 1000, 256, 5, None, None, ctypes.byref(c),
                                  ctypes.byref(c)) == NULL
    # a large k keeps 1,024-row chunks (the fused merge could not hold 251 x 512
    # candidates), so both plans coincide
    assert lt.workspace_bytes(1, 128256, 512) == lt.workspace_bytes(1, 128256, 512, chunk_rows=1024)


def test_status_strings():
    lib = lt._lib
    for s in range(10):
        assert lib.lmtopk_status_string(s)
    assert lib.lmtopk_status_string(99) == b"unknown status"


def _binary(**kw):
    a = dict(act_q=A, act_scale=A, wq=A, wscale=A, bias=None, M=1, V=1000, H=256, group=128,
             k=10, values=A, indices=A, ws=A, ws_bytes=BIG, opt=None, stream=None)
    a.update(kw)
    return lt._lib.lmtopk_binary(a["act_q"], a["act_scale"], a["wq"], a["wscale"], a["bias"],
                                 a["M"], a["V"], a["H"], a["group"], a["k"], a["values"],
                                 a["indices"], a["ws"], a["ws_bytes"], a["opt"], a["stream"])


def _dense(**kw):
    a = dict(hidden=A, weight=A, dtype=0, bias=None, M=2, V=1000, H=256, k=10, values=A,
             indices=A, ws=A, ws_bytes=BIG, opt=None, stream=None)
    a.update(kw)
    return lt._lib.lmtopk_dense(a["hidden"], a["weight"], a["dtype"], a["bias"], a["M"], a["V"],
                                a["H"], a["k"], a["values"], a["indices"], a["ws"],
                                a["ws_bytes"], a["opt"], a["stream"])


def _select(**kw):
    a = dict(logits=A, M=1, V=1000, ld=1000, k=10, values=A, indices=A, ws=A, ws_bytes=BIG,
             opt=None, stream=None)
    a.update(kw)
    return lt._lib.lmtopk_select(a["logits"], a["M"], a["V"], a["ld"], a["k"], a["values"],
                                 a["indices"], a["ws"], a["ws_bytes"], a["opt"], a["stream"])


_KEEP = []


def opt(chunk_rows=0, reserved=0, lse=None, allowed=None, sampling=None):
    sp = ctypes.pointer(sampling) if sampling is not None else None
    o = lt._Options(chunk_rows, reserved, None, lse, allowed, sp)
    _KEEP.append((o, sampling))
    return ctypes.byref(o)


def smp(**kw):
    c = lt._SamplingC()
    c.temperature, c.top_k, c.top_p, c.min_p = 1.0, 0, 1.0, 0.0
    c.tokens = A
    for key, v in kw.items():
        setattr(c, key, v)
    return c


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs a C compiler")
def test_struct_layouts_match_the_header():
    """offsetof of every field, compiled from include/lmtopk.h, equals the
    binding's ctypes layout."""
    fields = {"lmtopk_options": lt._Options, "lmtopk_sampling": lt._SamplingC}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "lmtopk.h"', "int main(void) {"]
    for cname, py in fields.items():
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines.append("return 0; }")
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "l.c"), os.path.join(d, "l")
        open(src, "w").write("\n".join(lines))
        subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), src, "-o", exe],
                       check=True)
        out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split("\n")
    got = {tuple(l.split()[:2]): int(l.split()[2]) for l in out if l}
    for cname, py in fields.items():
        assert got[(cname, "size")] == ctypes.sizeof(py)
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)


@pytest.mark.parametrize("entry", ["binary", "dense", "select"])
def test_sampling_arguments_are_checked_before_any_launch(entry):
    call = {"binary": _binary, "dense": _dense, "select": _select}[entry]
    assert call(opt=opt(sampling=smp(tokens=None))) == NULL
    assert call(opt=opt(sampling=smp(tokens=ODD))) == ALIGN
    assert call(opt=opt(sampling=smp(kept=ODD))) == ALIGN
    assert call(opt=opt(sampling=smp(temperature_rows=ODD))) == ALIGN
    assert call(opt=opt(sampling=smp(offset_device=ODD))) == ALIGN
    assert call(opt=opt(sampling=smp(top_k=11))) == OPTIONS      # above the call's k = 10


def test_workspace_init_rejects():
    lib = lt._lib
    assert lib.lmtopk_workspace_init(None, 256, None) == NULL
    assert lib.lmtopk_workspace_init(ODD, 256, None) == ALIGN
    assert lib.lmtopk_workspace_init(A, 0, None) == OK   # nothing to fill, nothing launched


@pytest.mark.parametrize("entry", ["binary", "dense", "select"])
def test_misaligned_lse_or_bitmask_is_rejected_before_any_launch(entry):
    call = {"binary": _binary, "dense": _dense, "select": _select}[entry]
    assert call(opt=opt(lse=ODD)) == ALIGN
    assert call(opt=opt(allowed=ODD)) == ALIGN


@pytest.mark.parametrize("kw,code", [
    (dict(act_q=None), NULL), (dict(wscale=None), NULL), (dict(values=None), NULL),
    (dict(M=0), SHAPE), (dict(M=9), SHAPE), (dict(V=0), SHAPE), (dict(V=1 << 31), SHAPE),
    (dict(H=0), SHAPE), (dict(M=8, H=8320), SHAPE),
    (dict(k=0), K), (dict(k=2049, V=5000), K), (dict(k=11, V=10), K),
    (dict(group=64), GROUP), (dict(H=200), GROUP),
    (dict(act_q=ODD), ALIGN), (dict(wq=ODD), ALIGN), (dict(bias=ODD), ALIGN), (dict(values=ODD), ALIGN),
    (dict(ws=None), WORKSPACE), (dict(ws_bytes=16), WORKSPACE),
    (dict(opt=opt(100)), OPTIONS), (dict(opt=opt(4096)), OPTIONS), (dict(opt=opt(8192)), OPTIONS), (dict(opt=opt(0, 1)), OPTIONS),
    (dict(M=3, opt=opt(2048)), OPTIONS), (dict(M=8, V=5000, opt=opt(2048)), OPTIONS),
])
def test_binary_rejects(kw, code):
    assert _binary(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(hidden=None), NULL), (dict(weight=None), NULL), (dict(indices=None), NULL),
    (dict(M=9), SHAPE), (dict(H=0), SHAPE), (dict(k=0), K), (dict(dtype=2), DTYPE),
    (dict(H=6), ALIGN), (dict(H=4, dtype=1), ALIGN), (dict(weight=ODD), ALIGN),
    (dict(ws_bytes=0), WORKSPACE), (dict(opt=opt(-64)), OPTIONS),
])
def test_dense_rejects(kw, code):
    assert _dense(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(logits=None), NULL), (dict(ld=999), SHAPE), (dict(M=0), SHAPE), (dict(k=1001), K),
    (dict(logits=ODD), ALIGN), (dict(ws=None), WORKSPACE), (dict(opt=opt(3000)), OPTIONS),
])
def test_select_rejects(kw, code):
    assert _select(**kw) == code


def test_pack_and_size_query_rejects():
    lib = lt._lib
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.lmtopk_packed_bytes(10, 128, 128, None, ctypes.byref(b)) == NULL
    assert lib.lmtopk_packed_bytes(0, 128, 128, ctypes.byref(a), ctypes.byref(b)) == SHAPE
    assert lib.lmtopk_packed_bytes(10, 130, 128, ctypes.byref(a), ctypes.byref(b)) == GROUP
    assert lib.lmtopk_pack_binary(None, 0, 10, 128, 128, A, A, None) == NULL
    assert lib.lmtopk_pack_binary(A, 5, 10, 128, 128, A, A, None) == DTYPE
    assert lib.lmtopk_pack_binary(A, 0, 10, 100, 128, A, A, None) == GROUP
    assert lib.lmtopk_pack_binary(A, 0, 10, 128, 128, ODD, A, None) == ALIGN
    n = ctypes.c_size_t()
    assert lib.lmtopk_workspace_bytes(1, 100, 0, None, ctypes.byref(n)) == K
    assert lib.lmtopk_workspace_bytes(1, 100, 5, opt(65), ctypes.byref(n)) == OPTIONS
    assert lib.lmtopk_workspace_bytes(1, 100, 5, None, None) == NULL


def test_python_binding_checks_before_the_library():
    import torch
    with pytest.raises((ValueError, TypeError)):
        lt.lm_head_topk_binary(torch.zeros(1, 128, dtype=torch.int8), torch.ones(1),
                               torch.zeros(16, dtype=torch.uint8), torch.zeros(4), k=1,
                               vocab_size=1)
    with pytest.raises(ValueError):
        lt.topk_logits(torch.zeros(2, 10), 3)
