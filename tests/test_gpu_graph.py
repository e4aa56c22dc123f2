"""Calls captured in one HIP graph and replayed, against the oracle (GPU).

lm-head-topk page, section "Correctness": repeated calls are bitwise
identical.  A captured call keeps nothing of its own between replays except
the workspace's completion counter, which every call leaves at zero; this
test replays a graph of several calls (a fused binary call, a selection whose
candidates need separate merge launches, a call with a log-sum-exp output
and a bitmask, two geometries sharing one workspace, a token draw whose
offset is read from device memory) four times, with eager work between the
replays, and checks every replay against the oracle.
"""

import numpy as np
import pytest
import torch

import oracle
import synthetic
from parity import assert_select_exact, binary_eps_fn, check_draw, compare_end_to_end

pytestmark = pytest.mark.gpu

import lm_head_projection_amd as lt  # noqa: E402


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def test_graph_replays_match_the_oracle():
    torch.cuda.set_device(0)
    # 1. fused binary call (config-2 shape, two rows, bias), k = 50
    M, H, V, k = 2, 2048, 32001, 50
    W = synthetic.dense_head(V, H, 5)
    act_q, act_scale = synthetic.quantize_rows_int8(synthetic.hidden_rows(M, H, 5))
    bias = synthetic.bias_vector(V, 5)
    signs, scales = oracle.pack_logical(W)
    Lb = oracle.project_binary(act_q, act_scale, signs, scales, bias)
    wq, ws = lt.pack_binary(dev(W))
    d_aq, d_as, d_b = dev(act_q), dev(act_scale), dev(bias)
    ws_b = lt.new_workspace(M, V, k)
    out_b = (torch.empty((M, k), device="cuda"), torch.empty((M, k), dtype=torch.int64, device="cuda"))
    # 2. selection needing separate merge launches (k = 1,024 over 248,320)
    x2 = synthetic.random_logits(2, 248320, seed=41, ties=500)
    d_x2 = dev(x2)
    ws_2 = lt.new_workspace(2, 248320, 1024)
    out_2 = (torch.empty((2, 1024), device="cuda"), torch.empty((2, 1024), dtype=torch.int64, device="cuda"))
    # 3. lse and bitmask on the selection path
    x3 = synthetic.random_logits(3, 50000, seed=42)
    rng = np.random.default_rng(42)
    allowed = rng.random((3, 50000)) < 0.5
    pad = np.zeros((3, ((50000 + 31) // 32) * 32), dtype=bool)
    pad[:, :50000] = allowed
    bm = np.packbits(pad, axis=1, bitorder="little").view("<i4")
    x3m = oracle.apply_allowed(x3, bm)
    d_x3, d_bm = dev(x3), dev(bm)
    lse3 = torch.empty(3, device="cuda")
    out_3 = (torch.empty((3, 64), device="cuda"), torch.empty((3, 64), dtype=torch.int64, device="cuda"))
    # 4. two geometries sharing one workspace
    x4a = synthetic.random_logits(1, 248320, seed=43)
    x4b = synthetic.random_logits(4, 7000, seed=44, ties=30)
    d_x4a, d_x4b = dev(x4a), dev(x4b)
    ws_4 = lt.new_workspace(4, 248320, 100)
    assert ws_4.numel() >= max(lt.workspace_bytes(1, 248320, 50), lt.workspace_bytes(4, 7000, 100))
    out_4a = (torch.empty((1, 50), device="cuda"), torch.empty((1, 50), dtype=torch.int64, device="cuda"))
    out_4b = (torch.empty((4, 100), device="cuda"), torch.empty((4, 100), dtype=torch.int64, device="cuda"))
    # 5. a draw with its offset in device memory
    x5 = synthetic.random_logits(4, 30000, seed=45)
    d_x5 = dev(x5)
    offset = torch.zeros(1, dtype=torch.int64, device="cuda")
    smp = lt.Sampling(0.8, 40, 0.9, 0.0, seed=77, offset=offset)
    ws_5 = lt.new_workspace(4, 30000, 40)
    out_5 = (torch.empty((4, 40), device="cuda"), torch.empty((4, 40), dtype=torch.int64, device="cuda"))
    tok5 = torch.empty(4, dtype=torch.int64, device="cuda")
    kept5 = torch.empty(4, dtype=torch.int32, device="cuda")

    def calls():
        lt.lm_head_topk_binary(d_aq, d_as, wq, ws, bias=d_b, k=k, out=out_b, workspace=ws_b)
        lt.topk_logits(d_x2, 1024, out=out_2, workspace=ws_2)
        lt.topk_logits(d_x3, 64, out=out_3, workspace=ws_2, lse=lse3, allowed=d_bm)
        lt.topk_logits(d_x4a, 50, out=out_4a, workspace=ws_4)
        lt.topk_logits(d_x4b, 100, out=out_4b, workspace=ws_4)
        lt.topk_logits(d_x5, 40, out=out_5, workspace=ws_5, sampling=smp, tokens=tok5, kept=kept5)

    # eager once (the allocator and the library are warm before capture)
    calls()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    eps_b = binary_eps_fn(act_q, act_scale, lambda ix: scales[ix], bias, H // 128)
    noise = torch.randn(512, 512, device="cuda")
    for rep in range(4):
        for t in (*out_b, *out_2, *out_3, *out_4a, *out_4b, tok5, kept5, lse3):
            t.fill_(-7)
        offset.fill_(rep)
        g.replay()
        # eager work of the program's own between replays
        noise = noise @ noise.T / 512.0
        lt.topk_logits(d_x4b, 10)
        torch.cuda.synchronize()
        compare_end_to_end(Lb, out_b[0].cpu().numpy(), out_b[1].cpu().numpy(), k, 1e-2, eps_b)
        assert_select_exact(x2, out_2[0].cpu().numpy(), out_2[1].cpu().numpy(), 1024)
        assert_select_exact(x3m, out_3[0].cpu().numpy(), out_3[1].cpu().numpy(), 64)
        want = oracle.logsumexp_rows(x3m)
        assert np.allclose(lse3.cpu().numpy(), want, rtol=0, atol=1e-5 + 2.0**-20 * np.abs(want).max())
        assert_select_exact(x4a, out_4a[0].cpu().numpy(), out_4a[1].cpu().numpy(), 50)
        assert_select_exact(x4b, out_4b[0].cpu().numpy(), out_4b[1].cpu().numpy(), 100)
        t5, k5 = tok5.cpu().numpy(), kept5.cpu().numpy()
        for m in range(4):
            r = oracle.sample_row(x5[m], 40, 0.8, 40, 0.9, 0.0, 77, m, rep)
            r.update(seed=77, row=m, offset=rep)
            check_draw(r, t5[m], k5[m], 40, 0.9, 0.0, 40)
    del g
