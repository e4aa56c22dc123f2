"""Token draw over the top-k survivors against the oracle (GPU).

logits-processor page, section "API" (temperature, top_k, top_p, min_p per
row; a draw keyed by (seed, row, offset), deterministic and replayable),
section "Method" (the filters meet in one keep set; Gumbel-max over it) and
section "Correctness" (greedy and top_k = 1 give the argmax; the token lies in
the keep set; the distribution matches the filtered softmax; per-row
parameters are honoured; a bitmask is never violated).

Every GPU draw is compared with the oracle's draw for the same (seed, row,
offset): the keep-set size and the token must be the oracle's wherever its
decisions are clear of the fp32 allowance (tests/parity.py, check_draw).
"""

import math

import numpy as np
import pytest
import torch

import oracle
import synthetic
from parity import binary_eps_fn, check_draw

pytestmark = pytest.mark.gpu

import lm_head_projection_amd as lt  # noqa: E402


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def per_row(x, M):
    a = np.asarray(x)
    return np.broadcast_to(a, (M,)) if a.ndim == 0 else a


def oracle_rows(L, k, T, tk, tp, mp, seed, offset):
    M = L.shape[0]
    T, tk, tp, mp = (per_row(x, M) for x in (T, tk, tp, mp))
    out = []
    for m in range(M):
        r = oracle.sample_row(L[m], k, float(T[m]), int(tk[m]), float(tp[m]), float(mp[m]),
                              seed, m, offset)
        r.update(seed=seed, row=m, offset=offset)
        out.append(r)
    return out


def check_rows(L, k, T, tk, tp, mp, seed, offset, tokens, kept, eps_z=0.0):
    M = L.shape[0]
    rs = oracle_rows(L, k, T, tk, tp, mp, seed, offset)
    tk_, tp_, mp_ = (per_row(x, M) for x in (tk, tp, mp))
    relaxed = 0
    for m in range(M):
        relaxed += check_draw(rs[m], tokens[m], kept[m], int(tk_[m]), float(tp_[m]), float(mp_[m]),
                              k, eps_z=eps_z)
    return rs, relaxed


def select_draw(x, k, s, chunk_rows=0, allowed=None):
    M = x.shape[0]
    kept = torch.empty(M, dtype=torch.int32, device="cuda")
    v, i, t = lt.topk_logits(dev(x), k, chunk_rows=chunk_rows, sampling=s, kept=kept,
                             allowed=allowed)
    torch.cuda.synchronize()
    return v.cpu().numpy(), i.cpu().numpy(), t.cpu().numpy(), kept.cpu().numpy()


@pytest.mark.parametrize("T,tk,tp,mp", [
    (1.0, 0, 1.0, 0.0), (0.7, 50, 0.9, 0.0), (1.3, 20, 1.0, 0.05), (0.5, 0, 0.95, 0.1),
    (2.0, 3, 0.5, 0.0),
])
@pytest.mark.parametrize("k", [1, 50, 300])
def test_select_path_matches_oracle(T, tk, tp, mp, k):
    x = synthetic.random_logits(4, 30001, seed=31)
    tk = min(tk, k)
    relaxed = 0
    for seed, offset in ((0, 0), (7, 123), (2**40 + 3, 2**35 + 9)):
        v, i, t, kept = select_draw(x, k, lt.Sampling(T, tk, tp, mp, seed, offset))
        _, rl = check_rows(x, k, T, tk, tp, mp, seed, offset, t, kept)
        relaxed += rl
    assert relaxed <= 1


def test_per_row_parameters_from_device_arrays():
    M, V, k = 6, 20000, 64
    x = synthetic.random_logits(M, V, seed=32)
    T = np.array([0.0, 0.6, 1.0, 1.5, 0.9, -1.0], dtype=np.float32)
    tk = np.array([0, 10, 64, 5, 0, 3], dtype=np.int32)
    tp = np.array([1.0, 0.8, 0.95, 1.0, 0.3, 0.5], dtype=np.float32)
    mp = np.array([0.0, 0.0, 0.02, 0.2, 0.0, 0.0], dtype=np.float32)
    s = lt.Sampling(dev(T), dev(tk), dev(tp), dev(mp), seed=99, offset=5)
    v, i, t, kept = select_draw(x, k, s)
    check_rows(x, k, T.astype(np.float64), tk, tp.astype(np.float64), mp.astype(np.float64), 99, 5,
               t, kept)
    assert kept[0] == 1 and t[0] == i[0, 0] and kept[5] == 1 and t[5] == i[5, 0]


def test_greedy_and_top1_are_the_argmax_bit_exactly():
    x = synthetic.random_logits(8, 50000, seed=33, ties=40)  # frequent ties for the maximum
    first_max = [int(np.argmax(x[m])) for m in range(8)]
    for s in (lt.Sampling(0.0), lt.Sampling(1.0, top_k=1), lt.Sampling(0.8, top_p=0.0),
              lt.Sampling(-2.0, 5, 0.5, 0.1)):
        for k in (1, 10):
            if s.top_k > k:
                continue
            _, i, t, kept = select_draw(x, k, s)
            assert t.tolist() == first_max and kept.tolist() == [1] * 8
    _, i, t, kept = select_draw(x, 1, lt.Sampling(1.7, seed=3, offset=4))
    assert t.tolist() == first_max


def test_draws_over_offsets_match_oracle_and_the_filtered_softmax():
    """2,000 draws (offsets 0..1,999) of one row: each one is the oracle's
    draw (up to the fp32 allowance), none leaves the keep set, and the
    frequencies pass a chi-square test against the renormalized softmax."""
    scipy_stats = pytest.importorskip("scipy.stats")
    V, k = 5000, 16
    x = synthetic.random_logits(1, V, seed=34) * np.float32(0.6)
    T, tk, tp, mp = 0.9, 0, 0.9, 0.01
    s = lt.Sampling(T, tk, tp, mp, seed=2024, offset=torch.zeros(1, dtype=torch.int64, device="cuda"))
    tokens = torch.empty(1, dtype=torch.int64, device="cuda")
    kept = torch.empty(1, dtype=torch.int32, device="cuda")
    d_x = dev(x)
    draws = 2000
    got_t, got_k = [], []
    for off in range(draws):
        s.offset.fill_(off)
        lt.topk_logits(d_x, k, sampling=s, tokens=tokens, kept=kept)
        got_t.append(tokens.clone())
        got_k.append(kept.clone())
    torch.cuda.synchronize()
    got_t = torch.cat(got_t).cpu().numpy()
    got_k = torch.cat(got_k).cpu().numpy()
    assert len(set(got_k.tolist())) == 1
    r0 = oracle.sample_row(x[0], k, T, tk, tp, mp, 2024, 0, 0)
    n = int(got_k[0])
    keep = [int(v) for v in r0["indices"][:n]]
    relaxed = 0
    for off in range(draws):
        r = oracle.sample_row(x[0], k, T, tk, tp, mp, 2024, 0, off)
        r.update(seed=2024, row=0, offset=off)
        relaxed += check_draw(r, got_t[off], got_k[off], tk, tp, mp, k)
    assert relaxed <= 2
    counts = np.array([(got_t == t).sum() for t in keep], dtype=np.float64)
    assert counts.sum() == draws
    w = np.exp(r0["z"][:n] - r0["z"][0])
    expect = draws * w / w.sum()
    stat = float(np.sum((counts - expect) ** 2 / expect))
    assert stat < scipy_stats.chi2.ppf(1.0 - 1e-6, n - 1), (stat, counts, expect)


def test_draws_are_deterministic_and_keyed():
    x = synthetic.random_logits(8, 40000, seed=35)
    s = lt.Sampling(1.0, 0, 1.0, 0.0, seed=5, offset=17)
    t1 = select_draw(x, 200, s)[2]
    t2 = select_draw(x, 200, s)[2]
    t3 = select_draw(x, 200, s, chunk_rows=256)[2]
    assert np.array_equal(t1, t2) and np.array_equal(t1, t3)
    # another offset or seed redraws (200 kept tokens per row: a change in
    # some row is certain in practice)
    assert not np.array_equal(t1, select_draw(x, 200, lt.Sampling(1.0, 0, 1.0, 0.0, 5, 18))[2])
    assert not np.array_equal(t1, select_draw(x, 200, lt.Sampling(1.0, 0, 1.0, 0.0, 6, 17))[2])


def test_bitmask_is_never_violated():
    M, V, k = 4, 10000, 64
    x = synthetic.random_logits(M, V, seed=36)
    rng = np.random.default_rng(36)
    allowed = rng.random((M, V)) < 0.02  # ~200 allowed entries per row
    allowed[3] = False
    allowed[3, [7, 9000]] = True  # two allowed entries, fewer than k
    W = (V + 31) // 32
    padded = np.zeros((M, W * 32), dtype=bool)
    padded[:, :V] = allowed
    bm = np.packbits(padded, axis=1, bitorder="little").view("<i4")
    xm = oracle.apply_allowed(x, bm)
    for off in range(5):
        s = lt.Sampling(1.5, 0, 0.99, 0.0, seed=1, offset=off)
        v, i, t, kept = select_draw(x, k, s, allowed=dev(bm))
        for m in range(M):
            assert allowed[m, t[m]]
        check_rows(xm, k, 1.5, 0, 0.99, 0.0, 1, off, t, kept)
    assert set(t[3:4].tolist()) <= {7, 9000} and kept[3] <= 2


def test_two_level_merge_path_draws():
    # k = 1,024 over 248,320 entries: the candidates need separate merge launches
    x = synthetic.random_logits(2, 248320, seed=37) * np.float32(0.3)
    s = lt.Sampling(1.0, 0, 0.97, 0.0, seed=8, offset=1)
    v, i, t, kept = select_draw(x, 1024, s)
    check_rows(x, 1024, 1.0, 0, 0.97, 0.0, 8, 1, t, kept)


def test_lse_output_is_the_sampled_normaliser():
    x = synthetic.random_logits(3, 30000, seed=38)
    lse = torch.empty(3, dtype=torch.float32, device="cuda")
    for T in (1.0, 0.5):
        lt.topk_logits(dev(x), 20, lse=lse, sampling=lt.Sampling(T, top_p=0.9))
        torch.cuda.synchronize()
        want = oracle.logsumexp_rows(x.astype(np.float64) / T)
        assert np.allclose(lse.cpu().numpy(), want, rtol=0, atol=1e-5 + 2.0**-22 * np.abs(want).max() * 4)


@pytest.mark.parametrize("path,M,H,chunk_rows", [
    ("binary", 3, 1024, 0),
    # five rows, 1,024-row chunks, G = 16: one wave per tile, matrix-core sums
    ("binary", 5, 2048, 1024),
    ("dense", 3, 1024, 0),
])
def test_fused_paths_draw_like_the_oracle(path, M, H, chunk_rows):
    V, k = 32001, 50
    T, tk, tp, mp = 0.7, 40, 0.9, 0.0
    if path == "binary":
        W = synthetic.dense_head(V, H, 3)
        act_q, act_scale = synthetic.quantize_rows_int8(synthetic.hidden_rows(M, H, 3))
        bias = synthetic.bias_vector(V, 3)
        signs, scales = oracle.pack_logical(W)
        L = oracle.project_binary(act_q, act_scale, signs, scales, bias)
        wq, ws = lt.pack_binary(dev(W))
        eps = binary_eps_fn(act_q, act_scale, lambda ix: scales[ix], bias, H // 128)
        eps_z = max(float(eps(m, np.arange(V)).max()) for m in range(M)) / T
    else:
        W = synthetic.dense_head(V, H, 4)
        hid = synthetic.hidden_rows(M, H, 4)
        L = oracle.project_dense(hid, W)
        eps_z = float((H / 64 + 8) * 2.0**-24 * (np.abs(hid) @ np.abs(W).T).max()) / T
    for offset in range(4):
        s = lt.Sampling(T, tk, tp, mp, seed=12, offset=offset)
        kept = torch.empty(M, dtype=torch.int32, device="cuda")
        if path == "binary":
            v, i, t = lt.lm_head_topk_binary(dev(act_q), dev(act_scale), wq, ws, bias=dev(bias), k=k,
                                             sampling=s, kept=kept, chunk_rows=chunk_rows)
        else:
            v, i, t = lt.lm_head_topk_dense(dev(hid), dev(W), k=k, sampling=s, kept=kept)
        torch.cuda.synchronize()
        check_rows(L, k, T, tk, tp, mp, 12, offset, t.cpu().numpy(), kept.cpu().numpy(), eps_z=eps_z)


@pytest.mark.slow
def test_flagship_binary_draw():
    M, H, V, k = 1, 5120, 248320, 50
    W = synthetic.dense_head(V, H, 0)
    act_q, act_scale = synthetic.quantize_rows_int8(synthetic.hidden_rows(M, H, 0))
    wq, ws = lt.pack_binary(dev(W))
    signs, scales = np.empty((V, H), np.int8), np.empty((V, H // 128), np.float32)
    for v0 in range(0, V, 8192):
        signs[v0:v0 + 8192], scales[v0:v0 + 8192] = oracle.pack_logical(W[v0:v0 + 8192])
    del W
    L = oracle.project_binary(act_q, act_scale, signs, scales)
    eps = binary_eps_fn(act_q, act_scale, lambda ix: scales[ix], None, H // 128)
    T = 0.7
    eps_z = float(eps(0, np.arange(V)).max()) / T
    for offset in range(3):
        s = lt.Sampling(T, 50, 0.9, 0.0, seed=0, offset=offset)
        kept = torch.empty(1, dtype=torch.int32, device="cuda")
        v, i, t = lt.lm_head_topk_binary(dev(act_q), dev(act_scale), wq, ws, k=k, vocab_size=V,
                                         sampling=s, kept=kept)
        torch.cuda.synchronize()
        check_rows(L, k, T, 50, 0.9, 0.0, 0, offset, t.cpu().numpy(), kept.cpu().numpy(), eps_z=eps_z)
