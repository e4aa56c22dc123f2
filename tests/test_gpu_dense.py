"""Dense head (fp32 and bf16): GPU fused projection + top-k against the oracle.

lm-head-topk page, section "Usage" (dense entry point, kept as the
correctness reference) and section "Correctness" (rows 1 to 8, hidden 512 to
2,048, vocabularies 8,192 to 128,256, k 1 to 100, with and without bias;
values to 1e-5).
"""

import math

import numpy as np
import pytest
import torch

import oracle
import synthetic
from parity import compare_end_to_end, dense_eps_fn

pytestmark = pytest.mark.gpu

import lm_head_projection_amd as lt  # noqa: E402

RTOL_DENSE = 1e-5


def bf16_tensor(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def make_case(M, H, V, seed, dtype, with_bias):
    h32 = synthetic.hidden_rows(M, H, seed)
    w32 = synthetic.dense_head(V, H, seed)
    bias = synthetic.bias_vector(V, seed) if with_bias else None
    if dtype == "bf16":
        hb, wb = synthetic.f32_to_bf16_bits(h32), synthetic.f32_to_bf16_bits(w32)
        h_ref, w_ref = oracle.bf16_bits_to_f32(hb), oracle.bf16_bits_to_f32(wb)
        h_dev, w_dev = bf16_tensor(hb), bf16_tensor(wb)
    else:
        h_ref, w_ref = h32, w32
        h_dev, w_dev = torch.from_numpy(h32).cuda(), torch.from_numpy(w32).cuda()
    b_dev = torch.from_numpy(bias).cuda() if bias is not None else None
    return h_ref, w_ref, bias, h_dev, w_dev, b_dev


def check(M, H, V, k, seed, dtype, with_bias, chunk_rows=0):
    h_ref, w_ref, bias, h_dev, w_dev, b_dev = make_case(M, H, V, seed, dtype, with_bias)
    v, i = lt.lm_head_topk_dense(h_dev, w_dev, k=k, bias=b_dev, chunk_rows=chunk_rows)
    torch.cuda.synchronize()
    L = oracle.project_dense(h_ref, w_ref, bias)
    eps = dense_eps_fn(h_ref, lambda ix: w_ref[ix], bias, H)
    return compare_end_to_end(L, v.cpu().numpy(), i.cpu().numpy(), k, RTOL_DENSE, eps)


def test_dense_fp32_small_config():
    """Dense fp32 head, M=1, H=512, V=8,192 (4 chunks of 2,048), k=10, no bias."""
    check(1, 512, 8192, 10, 0, "f32", False, chunk_rows=2048)
    check(1, 512, 8192, 10, 0, "f32", False)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M,H,V,k,with_bias", [
    (1, 512, 8192, 1, False), (3, 1024, 32001, 50, True), (8, 2048, 8192, 100, False),
    (2, 768, 40000, 64, True), (5, 2048, 16411, 17, True),
])
def test_dense_grid(dtype, M, H, V, k, with_bias):
    check(M, H, V, k, 1, dtype, with_bias)


@pytest.mark.slow
def test_dense_bf16_large_vocab():
    check(1, 4096, 128256, 50, 2, "bf16", True)


def test_dense_one_hot_gives_the_column_bitwise():
    V, H = 5000, 512
    w = synthetic.dense_head(V, H, 3)
    bias = synthetic.bias_vector(V, 3)
    for j in (0, 300, 511):
        h = np.zeros((1, H), dtype=np.float32)
        h[0, j] = 1.0
        v, i = lt.lm_head_topk_dense(torch.from_numpy(h).cuda(), torch.from_numpy(w).cuda(), k=20,
                                     bias=torch.from_numpy(bias).cuda())
        torch.cuda.synchronize()
        col = (w[:, j] + bias).astype(np.float32)  # one product of 1.0 and one add: exact in fp32
        ov, oi = oracle.topk_stable(col, 20)
        assert np.array_equal(i.cpu().numpy()[0], oi)
        assert np.array_equal(v.cpu().numpy()[0].view(np.uint32), ov.view(np.uint32))


def test_dense_repeat_and_chunk_invariance():
    h_ref, w_ref, bias, h_dev, w_dev, b_dev = make_case(4, 1024, 20000, 4, "bf16", True)
    v0, i0 = lt.lm_head_topk_dense(h_dev, w_dev, k=50, bias=b_dev)
    for c in (0, 256, 512, 2048, 0, 0):
        v, i = lt.lm_head_topk_dense(h_dev, w_dev, k=50, bias=b_dev, chunk_rows=c)
        assert torch.equal(i, i0) and torch.equal(v.view(torch.int32), v0.view(torch.int32))
    # a row alone gives the same bits as inside M=4
    for m in range(4):
        v1, i1 = lt.lm_head_topk_dense(h_dev[m:m + 1].contiguous(), w_dev, k=50, bias=b_dev)
        assert torch.equal(i1[0], i0[m]) and torch.equal(v1[0].view(torch.int32), v0[m].view(torch.int32))


@pytest.mark.slow
def test_dense_bf16_flagship_shape():
    """Dense bf16 head at the measured shape: M=1, H=5,120, V=248,320, k=50
    (lm-head-topk page, section "Measured": the bf16 comparison path)."""
    relaxed = check(1, 5120, 248320, 50, 0, "bf16", False)
    assert relaxed <= 2
