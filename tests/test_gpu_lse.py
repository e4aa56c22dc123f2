"""Row log-sum-exp returned beside the top-k: GPU against the oracle.

Selective Log Softmax page (log-probability = logit - log-sum-exp of the
row; section "Kernel design": per-slice maxima and sums, combined).  The
library reduces each wave of a chunk to a (max, sum) pair and combines them
in the final merge, fused or in a merge launch.

Tolerance.  On fp32 logits given as input (selection path) the only error is
fp32 evaluation: each exponential and product to a few ulp, and at most ~40
fp32 additions or roundings along any path of the reduction tree, so the sum
is off by a relative 40 * 2^-24 ~ 2.4e-6 and its log by as much absolutely;
the final M + log(S) adds one rounding of |lse|.  Bound used:
1e-5 + 2^-22 * |lse|.  When the library computes the logits itself, log-sum-
exp moves by at most the largest error of any logit (it is 1-Lipschitz in
the max norm), so the bound adds max_v eps_v from the end-to-end tests'
a-priori fp32 logit bounds.
"""

import numpy as np
import pytest
import torch

import oracle
import synthetic
from parity import binary_eps_fn, dense_eps_fn

pytestmark = pytest.mark.gpu

import lm_head_projection_amd as lt  # noqa: E402
from test_gpu_binary import Case  # noqa: E402


def lse_bound(ref, logit_eps=0.0):
    return 1e-5 + 2.0 ** -22 * np.abs(ref) + logit_eps


def assert_lse(got, ref, logit_eps=0.0):
    got = np.asarray(got, dtype=np.float64)
    for m in range(ref.shape[0]):
        if np.isinf(ref[m]):
            assert got[m] == ref[m], f"row {m}: {got[m]} vs {ref[m]}"
            continue
        err = abs(got[m] - ref[m])
        eps = logit_eps[m] if np.ndim(logit_eps) else logit_eps
        assert err <= lse_bound(ref[m], eps), f"row {m}: lse {got[m]!r} vs {ref[m]!r} (err {err:.3e})"


def run_select_lse(x, k, chunk_rows=0):
    t = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    lse = torch.empty(x.shape[0], dtype=torch.float32, device="cuda")
    v, i = lt.topk_logits(t, k, chunk_rows=chunk_rows, lse=lse)
    v0, i0 = lt.topk_logits(t, k, chunk_rows=chunk_rows)
    torch.cuda.synchronize()
    # asking for the normalizer leaves the top-k unchanged, bit for bit
    assert torch.equal(i, i0) and torch.equal(v.view(torch.int32), v0.view(torch.int32))
    return lse.cpu().numpy(), v.cpu().numpy()


@pytest.mark.parametrize("M,V,k,chunk_rows", [
    (1, 1, 1, 0), (2, 1000, 7, 0), (3, 32001, 50, 0), (2, 40000, 64, 256),
    (3, 248320, 50, 0),      # flagship vocabulary, merge fused into the chunk launch
    (2, 248320, 1024, 0),    # two merge levels in merge launches
    (2, 100000, 100, 2048),
])
def test_select_path_lse(M, V, k, chunk_rows):
    x = synthetic.random_logits(M, V, seed=V + k, ties=0) * np.float32(4.0)
    got, _ = run_select_lse(x, k, chunk_rows)
    assert_lse(got, oracle.logsumexp_rows(x))


def test_select_path_lse_infinities_and_log_probs():
    V = 5000
    x = synthetic.random_logits(4, V, seed=9, ties=0)
    x[1, 1234] = np.inf          # an +inf logit: lse is +inf
    x[2, :] = -np.inf            # every logit -inf: lse is -inf
    x[3, ::3] = -np.inf          # a third of the row is -inf
    got, v = run_select_lse(x, 10)
    ref = oracle.logsumexp_rows(x)
    assert_lse(got, ref)
    # the top-k log-probabilities of a finite row, against the oracle's
    lp = v[0].astype(np.float64) - got[0]
    want = np.sort(x[0].astype(np.float64))[::-1][:10] - ref[0]
    assert np.allclose(lp, want, rtol=0, atol=lse_bound(ref[0]) + 1e-6)


@pytest.mark.parametrize("M,H,V,k", [(1, 1024, 32001, 50), (2, 2048, 40000, 64), (6, 512, 9000, 13)])
def test_binary_path_lse(M, H, V, k):
    c = Case(M, H, V, seed=M + V, with_bias=True)
    lse = torch.empty(M, dtype=torch.float32, device="cuda")
    v, i = lt.lm_head_topk_binary(c.d_act, c.d_scale, c.wq, c.ws, bias=c.d_bias, k=k,
                                  vocab_size=V, lse=lse)
    torch.cuda.synchronize()
    eps_fn = binary_eps_fn(c.act_q, c.act_scale, lambda ix: c.scales[ix], c.bias, c.G)
    all_rows = np.arange(V)
    logit_eps = np.array([eps_fn(m, all_rows).max() for m in range(M)])
    assert_lse(lse.cpu().numpy(), oracle.logsumexp_rows(c.L), logit_eps)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dense_path_lse(dtype):
    M, H, V, k = 3, 1024, 20000, 20
    h32 = synthetic.hidden_rows(M, H, 5)
    w32 = synthetic.dense_head(V, H, 5)
    bias = synthetic.bias_vector(V, 5)
    if dtype == "bf16":
        hb, wb = synthetic.f32_to_bf16_bits(h32), synthetic.f32_to_bf16_bits(w32)
        h_ref, w_ref = oracle.bf16_bits_to_f32(hb), oracle.bf16_bits_to_f32(wb)
        h_dev = torch.from_numpy(np.ascontiguousarray(hb).view(np.int16)).cuda().view(torch.bfloat16)
        w_dev = torch.from_numpy(np.ascontiguousarray(wb).view(np.int16)).cuda().view(torch.bfloat16)
    else:
        h_ref, w_ref = h32, w32
        h_dev, w_dev = torch.from_numpy(h32).cuda(), torch.from_numpy(w32).cuda()
    lse = torch.empty(M, dtype=torch.float32, device="cuda")
    lt.lm_head_topk_dense(h_dev, w_dev, k=k, bias=torch.from_numpy(bias).cuda(), lse=lse)
    torch.cuda.synchronize()
    L = oracle.project_dense(h_ref, w_ref, bias)
    eps_fn = dense_eps_fn(h_ref, lambda ix: w_ref[ix], bias, H)
    logit_eps = np.array([eps_fn(m, np.arange(V)).max() for m in range(M)])
    assert_lse(lse.cpu().numpy(), oracle.logsumexp_rows(L), logit_eps)


def test_lse_repeated_calls_bitwise_identical():
    x = synthetic.random_logits(2, 248320, seed=3, ties=0)
    a, _ = run_select_lse(x, 50)
    b, _ = run_select_lse(x, 50)
    assert np.array_equal(a.view(np.int32), b.view(np.int32))
