"""Grammar bitmask inside the fused call: GPU against the oracle.

logits-processor page, section "API": bit 1 = allowed, disallowed logits are
set to -inf.  The library applies the bitmask to each logit it forms (or
reads), so the result must equal the oracle's top-k (and log-sum-exp) of the
masked logits: bit-exact on the selection path, within the end-to-end
tolerances where the library forms the logits.  Masks: random densities,
fewer allowed entries than k (the rest are -inf, returned in index order),
whole chunks masked, bits past V set.
"""

import numpy as np
import pytest
import torch

import oracle
import synthetic
from parity import assert_select_exact, binary_eps_fn, compare_end_to_end, dense_eps_fn

pytestmark = pytest.mark.gpu

import lm_head_projection_amd as lt  # noqa: E402
from test_gpu_binary import RTOL_BINARY, Case  # noqa: E402
from test_gpu_lse import assert_lse  # noqa: E402


def make_mask(M, V, density, seed, pad_bits=True):
    rng = np.random.default_rng(seed)
    allowed = rng.random((M, V)) < density
    W = (V + 31) // 32
    padded = np.zeros((M, W * 32), dtype=bool)
    padded[:, :V] = allowed
    if pad_bits:
        padded[:, V:] = True  # bits past V are ignored
    return np.packbits(padded, axis=1, bitorder="little").view("<i4").copy()


def masked_select(x, bm, k, chunk_rows=0):
    t = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    lse = torch.empty(x.shape[0], dtype=torch.float32, device="cuda")
    v, i = lt.topk_logits(t, k, chunk_rows=chunk_rows, lse=lse, allowed=torch.from_numpy(bm).cuda())
    torch.cuda.synchronize()
    return v.cpu().numpy(), i.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("M,V,k,density,chunk_rows", [
    (2, 1000, 7, 0.5, 0),
    (3, 248320, 50, 0.5, 0),      # fused merge
    (2, 248320, 1024, 0.3, 0),    # two merge levels
    (2, 40000, 64, 0.02, 256),
    (1, 70000, 100, 0.001, 2048),  # about 70 allowed entries
])
def test_select_path_mask(M, V, k, density, chunk_rows):
    x = synthetic.random_logits(M, V, seed=V + k, ties=50)
    bm = make_mask(M, V, density, seed=k)
    v, i, lse = masked_select(x, bm, k, chunk_rows)
    xm = oracle.apply_allowed(x, bm)
    assert_select_exact(xm, v, i, k)
    assert_lse(lse, oracle.logsumexp_rows(xm))


def test_select_path_fewer_allowed_than_k_and_masked_chunks():
    M, V, k = 3, 9000, 40
    x = synthetic.random_logits(M, V, seed=5, ties=0)
    bm = make_mask(M, V, 0.0, seed=1)
    allowed = np.zeros((M, V), dtype=bool)
    allowed[0, [3, 4000, 8999, 17]] = True      # four allowed entries
    allowed[1, 2048:4096] = True                # only one chunk-sized block allowed
    allowed[2, :] = True
    allowed[2, 1024:6144] = False               # whole chunks masked
    W = (V + 31) // 32
    padded = np.zeros((M, W * 32), dtype=bool)
    padded[:, :V] = allowed
    bm = np.packbits(padded, axis=1, bitorder="little").view("<i4").copy()
    v, i, lse = masked_select(x, bm, k)
    xm = oracle.apply_allowed(x, bm)
    assert_select_exact(xm, v, i, k)
    # row 0: its four allowed entries by value, then -inf entries from index 0 up
    assert set(i[0, :4].tolist()) == {3, 17, 4000, 8999}
    assert np.all(v[0, 4:] == -np.inf)
    rest = [j for j in range(V) if j not in (3, 17, 4000, 8999)][: k - 4]
    assert i[0, 4:].tolist() == rest
    assert_lse(lse, oracle.logsumexp_rows(xm))


@pytest.mark.parametrize("M,H,V,k", [(1, 1024, 32001, 50), (5, 512, 9000, 13), (2, 2048, 20000, 300)])
def test_binary_path_mask(M, H, V, k):
    c = Case(M, H, V, seed=M + H, with_bias=True)
    bm = make_mask(M, V, 0.4, seed=V)
    lse = torch.empty(M, dtype=torch.float32, device="cuda")
    v, i = lt.lm_head_topk_binary(c.d_act, c.d_scale, c.wq, c.ws, bias=c.d_bias, k=k, vocab_size=V,
                                  lse=lse, allowed=torch.from_numpy(bm).cuda())
    torch.cuda.synchronize()
    Lm = oracle.apply_allowed(c.L, bm)
    eps_fn = binary_eps_fn(c.act_q, c.act_scale, lambda ix: c.scales[ix], c.bias, c.G)
    compare_end_to_end(Lm, v.cpu().numpy(), i.cpu().numpy(), k, RTOL_BINARY, eps_fn)
    logit_eps = np.array([eps_fn(m, np.arange(V)).max() for m in range(M)])
    assert_lse(lse.cpu().numpy(), oracle.logsumexp_rows(Lm), logit_eps)


def test_dense_path_mask():
    M, H, V, k = 3, 768, 20000, 25
    h = synthetic.hidden_rows(M, H, 8)
    w = synthetic.dense_head(V, H, 8)
    bm = make_mask(M, V, 0.25, seed=8)
    v, i = lt.lm_head_topk_dense(torch.from_numpy(h).cuda(), torch.from_numpy(w).cuda(), k=k,
                                 allowed=torch.from_numpy(bm).cuda())
    torch.cuda.synchronize()
    Lm = oracle.apply_allowed(oracle.project_dense(h, w, None), bm)
    eps_fn = dense_eps_fn(h, lambda ix: w[ix], None, H)
    compare_end_to_end(Lm, v.cpu().numpy(), i.cpu().numpy(), k, 1e-5, eps_fn)


def test_all_allowed_mask_changes_nothing():
    M, V, k = 2, 50000, 50
    x = synthetic.random_logits(M, V, seed=2, ties=10)
    t = torch.from_numpy(x).cuda()
    bm = torch.full((M, (V + 31) // 32), -1, dtype=torch.int32, device="cuda")
    v0, i0 = lt.topk_logits(t, k)
    v1, i1 = lt.topk_logits(t, k, allowed=bm)
    torch.cuda.synchronize()
    assert torch.equal(i0, i1) and torch.equal(v0.view(torch.int32), v1.view(torch.int32))
