"""lmtopk_binary_noalloc (the binary entry point that allocates nothing) gives
the same bits as lmtopk_binary, called through the C ABI (GPU).

Two calls in a row, the second with smaller sizes, so the shared scratch
array is reused with a different geometry; sizes beyond the array are
refused before any launch."""

import ctypes

import numpy as np
import pytest
import torch

import synthetic

pytestmark = pytest.mark.gpu

import lm_head_projection_amd as lt  # noqa: E402

WORKSPACE = 7


def _fn():
    f = lt._lib.lmtopk_binary_noalloc
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    f.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, i32, vp, vp,
                  ctypes.POINTER(lt._Options), vp]
    f.restype = ctypes.c_int
    return f


def _case(M, H, V, seed):
    W = synthetic.dense_head(V, H, seed)
    act_q, act_scale = synthetic.quantize_rows_int8(synthetic.hidden_rows(M, H, seed))
    bias = synthetic.bias_vector(V, seed)
    wq, ws = lt.pack_binary(torch.from_numpy(W).cuda())
    return (torch.from_numpy(act_q).cuda(), torch.from_numpy(act_scale).cuda(), wq, ws,
            torch.from_numpy(bias).cuda())


def _noalloc(f, case, M, V, H, k, lse=None):
    aq, sc, wq, ws, b = case
    vals = torch.empty((M, k), device="cuda")
    idx = torch.empty((M, k), dtype=torch.int64, device="cuda")
    o = lt._Options(0, 0, None, lse.data_ptr() if lse is not None else None, None, None)
    st = f(aq.data_ptr(), sc.data_ptr(), wq.data_ptr(), ws.data_ptr(), b.data_ptr(), M, V, H, 128,
           k, vals.data_ptr(), idx.data_ptr(), ctypes.byref(o),
           torch.cuda.current_stream().cuda_stream)
    assert st == 0, st
    return vals, idx


def test_noalloc_matches_the_workspace_entry_point():
    f = _fn()
    big = (4, 2048, 60001, 100)
    small = (1, 1024, 20001, 10)
    two_levels = (2, 1024, 60001, 512)  # 59 x 512 candidates per row: the key histogram
    for (M, H, V, k), seed in ((big, 1), (small, 2), (two_levels, 3)):
        case = _case(M, H, V, seed)
        lse_a = torch.empty(M, device="cuda")
        lse_b = torch.empty(M, device="cuda")
        va, ia = _noalloc(f, case, M, V, H, k, lse_a)
        aq, sc, wq, ws, b = case
        vb, ib = lt.lm_head_topk_binary(aq, sc, wq, ws, bias=b, k=k, lse=lse_b)
        torch.cuda.synchronize()
        assert torch.equal(ia, ib)
        assert torch.equal(va.view(torch.int32), vb.view(torch.int32))
        assert torch.equal(lse_a.view(torch.int32), lse_b.view(torch.int32))
        # the same call again on the shared scratch: the same bits
        va2, ia2 = _noalloc(f, case, M, V, H, k)
        torch.cuda.synchronize()
        assert torch.equal(ia2, ia) and torch.equal(va2.view(torch.int32), va.view(torch.int32))


def test_noalloc_refuses_sizes_beyond_its_scratch():
    f = _fn()
    # 8 rows, k = 1,024 over 248,320 entries need about 17 MB of workspace
    assert lt.workspace_bytes(8, 248320, 1024) > (8 << 20)
    o = lt._Options(0, 0, None, None, None, None)
    A = 4096  # never dereferenced: the call is refused on the host
    st = f(A, A, A, A, None, 8, 248320, 5120, 128, 1024, A, A, ctypes.byref(o), None)
    assert st == WORKSPACE
