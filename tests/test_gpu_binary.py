"""Binary head: GPU pack and fused projection + top-k against the oracle.

lm-head-topk page, section "Usage" (binary entry point: int8 activations with
a per-row scale, signs with per-128-group scales, optional bias), section
"Correctness" (binary values to 1e-2 against a dequantized reference, exact
indices, k = 1 is the argmax, ragged final chunk, every winner planted in one
chunk, deterministic) and section "Requirements and limits" (offline
packing; k up to 2,048).
"""

import numpy as np
import pytest
import torch

import oracle
import synthetic
from parity import binary_eps_fn, binary_logit_f32, compare_end_to_end

pytestmark = pytest.mark.gpu

import lm_head_projection_amd as lt  # noqa: E402

RTOL_BINARY = 1e-2


class Case:
    """One binary-head workload: host arrays for the oracle, device arrays for the library."""

    def __init__(self, M, H, V, seed=0, with_bias=False, W=None, bias=None, act=None):
        self.M, self.H, self.V, self.G = M, H, V, H // 128
        self.W = synthetic.dense_head(V, H, seed) if W is None else W
        if act is None:
            x = synthetic.hidden_rows(M, H, seed)
            self.act_q, self.act_scale = synthetic.quantize_rows_int8(x)
        else:
            self.act_q, self.act_scale = act
        if bias is None and with_bias:
            bias = synthetic.bias_vector(V, seed)
        self.bias = bias
        self.signs, self.scales = self._oracle_pack()
        wd = torch.from_numpy(self.W).cuda()
        self.wq, self.ws = lt.pack_binary(wd)
        del wd
        self.d_act = torch.from_numpy(self.act_q).cuda()
        self.d_scale = torch.from_numpy(self.act_scale).cuda()
        self.d_bias = torch.from_numpy(self.bias).cuda() if self.bias is not None else None
        self._L = None

    def _oracle_pack(self):
        signs = np.empty((self.V, self.H), dtype=np.int8)
        scales = np.empty((self.V, self.G), dtype=np.float32)
        for v0 in range(0, self.V, 8192):
            s, sc = oracle.pack_logical(self.W[v0:v0 + 8192])
            signs[v0:v0 + 8192], scales[v0:v0 + 8192] = s, sc
        return signs, scales

    @property
    def L(self):
        if self._L is None:
            self._L = oracle.project_binary(self.act_q, self.act_scale, self.signs, self.scales,
                                            self.bias)
        return self._L

    def run(self, k, rows=None, chunk_rows=0, act_scale=None, act_q=None):
        aq = self.d_act if rows is None else self.d_act[rows].contiguous()
        sc = self.d_scale if rows is None else self.d_scale[rows].contiguous()
        if act_scale is not None:
            sc = act_scale
        if act_q is not None:
            aq = act_q
        v, i = lt.lm_head_topk_binary(aq, sc, self.wq, self.ws, bias=self.d_bias, k=k,
                                      vocab_size=self.V, chunk_rows=chunk_rows)
        torch.cuda.synchronize()
        return v, i

    def check(self, k, rows=None, chunk_rows=0):
        v, i = self.run(k, rows, chunk_rows)
        rsel = slice(None) if rows is None else rows
        L = self.L[rsel]
        eps = binary_eps_fn(self.act_q[rsel], self.act_scale[rsel], lambda ix: self.scales[ix],
                            self.bias, self.G)
        relaxed = compare_end_to_end(L, v.cpu().numpy(), i.cpu().numpy(), k, RTOL_BINARY, eps)
        return v, i, relaxed


def assert_pack_matches(case):
    s_gpu, sc_gpu = oracle.unpack_layout_bytes(case.wq.cpu().numpy(), case.ws.cpu().numpy(),
                                               case.V, case.H)
    assert np.array_equal(s_gpu, case.signs), "sign bits differ from the oracle pack"
    ulp = np.abs(sc_gpu.view(np.int32).astype(np.int64) - case.scales.view(np.int32).astype(np.int64))
    assert ulp.max() <= 1, f"group scales differ by {ulp.max()} ulp"
    # padding rows and padding groups are zero
    T, G = -(-case.V // 64), case.G
    wq = case.wq.cpu().numpy().view(np.uint32).reshape(T, G, 64, 4)
    ws = case.ws.cpu().numpy().reshape(T, -1, 64, 4)
    r_last = case.V - (T - 1) * 64
    assert not wq[T - 1, :, r_last:, :].any() and not ws[T - 1, :, r_last:, :].any()
    gq = ws.transpose(0, 2, 1, 3).reshape(T * 64, -1)
    assert not gq[:, G:].any()


# ---------------------------------------------------------------------------
# pack
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("V,H", [(1, 128), (63, 128), (65, 640), (1000, 384), (32001, 2048)])
def test_pack_fp32_matches_oracle(V, H):
    assert_pack_matches(Case(1, H, V, seed=V))


@pytest.mark.parametrize("V,H", [(130, 256), (5000, 1024)])
def test_pack_bf16_matches_oracle(V, H):
    W = synthetic.dense_head(V, H, 5)
    bits = synthetic.f32_to_bf16_bits(W)
    W_ref = oracle.bf16_bits_to_f32(bits)
    wq, ws = lt.pack_binary(torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16))
    s_gpu, sc_gpu = oracle.unpack_layout_bytes(wq.cpu().numpy(), ws.cpu().numpy(), V, H)
    s, sc = oracle.pack_logical(W_ref)
    assert np.array_equal(s_gpu, s)
    assert np.abs(sc_gpu.view(np.int32).astype(np.int64) - sc.view(np.int32).astype(np.int64)).max() <= 1


def test_pack_signed_zero_and_golden_layout():
    import json, os
    with open(os.path.join(os.path.dirname(__file__), "golden", "layout_v1_tiny.json")) as f:
        g = json.load(f)
    from test_oracle_pins import _golden_head
    W = _golden_head(g)
    wq, ws = lt.pack_binary(torch.from_numpy(W).cuda())
    words = wq.cpu().numpy().view(np.uint32).reshape(-1)
    expect = np.zeros(g["total_words"], dtype=np.uint32)
    for k, v in g["expected_words"].items():
        expect[int(k)] = int(v, 16)
    assert np.array_equal(words, expect)
    sc = ws.cpu().numpy().reshape(-1)
    assert sc[257] == 3.0 and sc[256] == 0.0 and sc[4] == 2.0 and sc[252] == 0.5


# ---------------------------------------------------------------------------
# small and edge shapes
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,H,V,k,with_bias", [
    (1, 128, 1, 1, False), (1, 128, 40, 40, True), (2, 640, 65, 7, False),
    (3, 512, 1000, 100, True), (8, 2048, 8192, 1, False), (8, 8192, 3000, 64, True),
    (4, 1024, 32001, 50, True), (1, 384, 70000, 2048, False),
    # from two rows on (one row per lane) the group sums come from the matrix cores
    (5, 1280, 5000, 50, False), (6, 384, 2049, 13, True), (7, 2560, 9000, 300, False),
])
def test_binary_shapes(M, H, V, k, with_bias):
    Case(M, H, V, seed=M + H + V, with_bias=with_bias).check(k)


@pytest.mark.parametrize("M", [3, 6])  # bit planes, and activation bytes with dot4
def test_full_int8_range_including_minus_128(M):
    H, V = 1024, 5000
    rng = np.random.default_rng(4)
    act_q = rng.integers(-128, 128, size=(M, H)).astype(np.int8)
    act_q[0, :] = -128
    act_q[1, ::2] = 127
    act_q[M - 1, 1::2] = -128
    act_scale = np.array([1e-3, 2e-3, 0.5, 0.25, 4e-3, 1.0][:M], dtype=np.float32)
    c = Case(M, H, V, seed=3, act=(act_q, act_scale), with_bias=True)
    c.check(50)


@pytest.mark.parametrize("with_lse", [False, True])
@pytest.mark.parametrize("M", [2, 5, 8])
def test_rows_select_independently(M, with_lse):
    # The rows' small-k chunk selections share their barriers, and with 50 to
    # 256 chunks of 16 waves the rows' merges run side by side (one group of
    # waves per row, each row's log-sum-exp by its group's first wave).  Row 1
    # has zero activations, so all its logits are equal: every chunk stages
    # all of its rows, more than the small-k staging holds, and that row takes
    # the radix select while the other rows keep the small-k one; in the
    # merge it has more survivors than its group holds and is merged by the
    # whole workgroup afterwards.  Each row equals the oracle and, bit for
    # bit, its own result alone (M = 1).
    H, V, k = 1024, 32001, 50
    _, n_chunks, waves = lt.binary_plan(M, V, H, k)
    assert k <= n_chunks <= 256 and waves == 16, "sizes of the side-by-side merge"
    rng = np.random.default_rng(M)
    act_q = rng.integers(-128, 128, size=(M, H)).astype(np.int8)
    act_q[1, :] = 0
    act_scale = (rng.random(M).astype(np.float32) + 0.5) * np.float32(1e-2)
    c = Case(M, H, V, seed=11, act=(act_q, act_scale))

    def call(rows):
        aq, sc = c.d_act[rows].contiguous(), c.d_scale[rows].contiguous()
        lse = torch.empty(len(rows), device="cuda") if with_lse else None
        v, i = lt.lm_head_topk_binary(aq, sc, c.wq, c.ws, k=k, vocab_size=V, lse=lse)
        torch.cuda.synchronize()
        return v, i, lse

    v, i, lse = call(list(range(M)))
    eps = binary_eps_fn(c.act_q, c.act_scale, lambda ix: c.scales[ix], None, c.G)
    compare_end_to_end(c.L, v.cpu().numpy(), i.cpu().numpy(), k, RTOL_BINARY, eps)
    assert np.array_equal(i.cpu().numpy()[1], np.arange(k)), "equal logits: the lowest indices"
    if with_lse:
        want = oracle.logsumexp_rows(c.L)
        tol = 1e-5 + 2.0**-22 * np.abs(want) + np.array([eps(m, np.arange(V)).max() for m in range(M)])
        assert np.all(np.abs(lse.cpu().numpy() - want) <= tol)
    for m in (0, 1, M - 1):
        v1, i1, l1 = call([m])
        assert torch.equal(i1[0], i[m]) and torch.equal(v1[0].view(torch.int32), v[m].view(torch.int32))
        if with_lse:
            assert torch.equal(l1.view(torch.int32)[0], lse.view(torch.int32)[m])


# ---------------------------------------------------------------------------
# config 2: M=2, H=2048, V=32001 (ragged), k=50, planted and duplicate variants
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def cfg2():
    return Case(2, 2048, 32001, seed=0)


def test_cfg2_plain(cfg2):
    cfg2.check(50)


@pytest.mark.parametrize("C", [2048, 1024, 512, 256])
def test_cfg2_all_winners_planted_in_chunk7(cfg2, C):
    rows = np.arange(7 * C, 7 * C + 50)
    bias = synthetic.planted_bias(cfg2.V, rows, 5.0)
    c = Case(2, 2048, 32001, W=cfg2.W, act=(cfg2.act_q, cfg2.act_scale), bias=bias)
    # precondition: the oracle's top-50 of every row is exactly the planted rows
    for m in range(2):
        _, oi = oracle.topk_stable(c.L[m], 50)
        assert set(oi.tolist()) == set(rows.tolist())
    for chunk_rows in {C, 0}:
        v, i, _ = c.check(50, chunk_rows=chunk_rows)
        assert set(i.cpu().numpy()[0].tolist()) == set(rows.tolist())


def test_cfg2_duplicates_straddle_k(cfg2):
    k = 50
    W = cfg2.W.copy()
    _, oi = oracle.topk_stable(cfg2.L[0], cfg2.V)
    src = int(oi[k - 4])               # rank 46 (0-based): copies fill ranks 46..53
    rank = np.empty(cfg2.V, dtype=np.int64)
    rank[oi] = np.arange(cfg2.V)
    targets = []
    for start in (0, 4096, 9000, 15000, 21000, 27000, cfg2.V - 200):  # last: the ragged chunk
        j = start
        while rank[j] <= 1000 or j == src:
            j += 1
        targets.append(j)
    W[targets] = W[src]
    c = Case(2, 2048, 32001, W=W, act=(cfg2.act_q, cfg2.act_scale))
    dup = sorted([src] + targets)
    _, oi2 = oracle.topk_stable(c.L[0], k)
    assert list(oi2[k - 4:]) == dup[:4], "precondition: 4 of the 8 copies fill ranks 46..49"
    v, i, _ = c.check(k)
    gi = i.cpu().numpy()[0]
    gv = v.cpu().numpy()[0]
    assert list(gi[k - 4:]) == dup[:4]
    assert len(set(gv[k - 4:].view(np.uint32).tolist())) == 1  # bitwise equal logits
    for C in (256, 2048):
        v2, i2 = c.run(k, chunk_rows=C)
        assert torch.equal(i2, i) and torch.equal(v2.view(torch.int32), v.view(torch.int32))


def test_cfg2_invariants(cfg2):
    v0, i0 = cfg2.run(50)
    for _ in range(10):  # repeated calls are bitwise identical
        v, i = cfg2.run(50)
        assert torch.equal(i, i0) and torch.equal(v.view(torch.int32), v0.view(torch.int32))
    for C in (64, 256, 512, 1024, 2048):  # chunk size does not change a bit
        v, i = cfg2.run(50, chunk_rows=C)
        assert torch.equal(i, i0) and torch.equal(v.view(torch.int32), v0.view(torch.int32))
    for m in range(2):  # a row alone equals the same row inside M=2
        v, i = cfg2.run(50, rows=[m])
        assert torch.equal(i[0], i0[m]) and torch.equal(v[0].view(torch.int32), v0[m].view(torch.int32))
    # doubling act_scale doubles every value exactly (no bias), same indices
    v, i = cfg2.run(50, act_scale=cfg2.d_scale * 2)
    assert torch.equal(i, i0) and torch.equal(v, v0 * 2)
    # negating the activations and every sign leaves each logit bit for bit
    neg = Case(2, 2048, 32001, W=-cfg2.W, act=(cfg2.act_q, cfg2.act_scale))
    v, i = neg.run(50, act_q=(-cfg2.d_act.to(torch.int16)).to(torch.int8))
    assert torch.equal(i, i0) and torch.equal(v.view(torch.int32), v0.view(torch.int32))


def test_cfg2_k1_is_argmax(cfg2):
    v, i = cfg2.run(1)
    assert np.array_equal(i.cpu().numpy()[:, 0], np.argmax(cfg2.L, axis=1))


# ---------------------------------------------------------------------------
# config 3: M=1, H=4096, V=128,256, k=50, bias N(0, 0.1)
# ---------------------------------------------------------------------------
@pytest.mark.slow
def test_cfg3_bias():
    c = Case(1, 4096, 128256, seed=0, with_bias=True)
    assert_pack_matches(c)
    c.check(50)


# ---------------------------------------------------------------------------
# configs 4 and 5: V=248,320, H=5,120
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def flagship():
    return Case(8, 5120, 248320, seed=0)


@pytest.mark.slow
def test_cfg4_flagship_m1(flagship):
    v, i, relaxed = flagship.check(50, rows=[0])
    assert relaxed <= 2
    assert_documented_fp32_order(flagship, v, i, [0])


@pytest.mark.slow
@pytest.mark.parametrize("M", [1, 4, 8])
@pytest.mark.parametrize("k", [1, 50, 1024])
def test_cfg5_sweep_with_bias(flagship, M, k):
    if not hasattr(flagship, "with_bias_case"):
        flagship.with_bias_case = Case(8, 5120, 248320, W=flagship.W,
                                       act=(flagship.act_q, flagship.act_scale),
                                       bias=synthetic.bias_vector(248320, 0))
    c = flagship.with_bias_case
    rows = list(range(M))
    v, i, _ = c.check(k, rows=rows)
    if k == 1:
        assert np.array_equal(i.cpu().numpy()[:, 0], np.argmax(c.L[:M], axis=1))


# ---------------------------------------------------------------------------
# chunk sizes x optional outputs: every binary kernel instance that exists
# runs (2048-row chunks, four rows per lane, serve M <= 2; from three rows on
# the library refuses them), with one wave per tile (1,024 and 2,048 rows)
# and with two (up to 512 rows; the automatic size at V = 20,001); from two
# rows on, with one row per lane, the group sums come from the matrix cores
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def wide_case():
    return Case(8, 2048, 20001, seed=9, with_bias=True)


def _mask(M, V, seed):
    rng = np.random.default_rng(seed)
    allowed = rng.random((M, V)) < 0.5
    pad = np.zeros((M, ((V + 31) // 32) * 32), dtype=bool)
    pad[:, :V] = allowed
    return np.packbits(pad, axis=1, bitorder="little").view("<i4")


@pytest.mark.parametrize("extras", ["none", "lse_and_mask"])
@pytest.mark.parametrize("chunk_rows", [0, 1024, 2048])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 8])
def test_chunk_sizes_and_extras(wide_case, M, chunk_rows, extras):
    c, k = wide_case, 50
    rows = list(range(M))
    aq, sc = c.d_act[:M].contiguous(), c.d_scale[:M].contiguous()
    lse = torch.empty(M, device="cuda") if extras != "none" else None
    bm = _mask(M, c.V, M) if extras != "none" else None
    kw = dict(bias=c.d_bias, k=k, vocab_size=c.V, chunk_rows=chunk_rows, lse=lse,
              allowed=torch.from_numpy(bm).cuda() if bm is not None else None)
    if chunk_rows == 2048 and M > 2:
        with pytest.raises(lt.LmTopkError) as e:
            lt.lm_head_topk_binary(aq, sc, c.wq, c.ws, **kw)
        assert e.value.status == 8  # LMTOPK_ERR_OPTIONS
        return
    v, i = lt.lm_head_topk_binary(aq, sc, c.wq, c.ws, **kw)
    torch.cuda.synchronize()
    L = c.L[:M] if bm is None else oracle.apply_allowed(c.L[:M], bm)
    eps = binary_eps_fn(c.act_q[:M], c.act_scale[:M], lambda ix: c.scales[ix], c.bias, c.G)
    compare_end_to_end(L, v.cpu().numpy(), i.cpu().numpy(), k, RTOL_BINARY, eps)
    if lse is not None:
        want = oracle.logsumexp_rows(L)
        tol = 1e-5 + 2.0**-22 * np.abs(want) + np.array([eps(m, np.arange(c.V)).max() for m in range(M)])
        assert np.all(np.abs(lse.cpu().numpy() - want) <= tol)
    # the chunk size does not change a bit
    v0, i0 = lt.lm_head_topk_binary(aq, sc, c.wq, c.ws, **{**kw, "chunk_rows": 256})
    assert torch.equal(i0, i) and torch.equal(v0.view(torch.int32), v.view(torch.int32))


# ---------------------------------------------------------------------------
# the two accumulation chains (quads [0, Qh) and [Qh, Q), Qh = floor(Q / 2)):
# one wave running both (1,024 and 2,048-row chunks) and two waves sharing a
# tile (512 and 64-row chunks) give the same bits for every group count,
# including an empty first chain (G <= 3) and a partial last quad, with the
# bit planes (one row, or four rows per lane) and with the matrix cores
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("G", [1, 2, 3, 4, 5, 7, 8, 9, 12, 13, 16, 20, 24])
@pytest.mark.parametrize("M", [1, 2, 5])
def test_split_chains_bitwise_across_chunk_sizes(M, G):
    c = Case(M, 128 * G, 3001, seed=G, with_bias=True)
    v0, i0, _ = c.check(20, chunk_rows=1024)
    sizes = (512, 64, 2048) if M <= 2 else (512, 64)
    for C in sizes:
        v, i = c.run(20, chunk_rows=C)
        assert torch.equal(i, i0) and torch.equal(v.view(torch.int32), v0.view(torch.int32)), C


def assert_documented_fp32_order(c, v, i, rows, n=None):
    """The returned values are the header's fp32 formula (two fused
    multiply-add chains over the group dots, their sum, then the row scale
    and bias), evaluated exactly with one rounding per operation: bit for
    bit, on the first n entries of each row."""
    v, i = v.cpu().numpy(), i.cpu().numpy()
    for r, m in enumerate(rows):
        a = c.act_q[m].astype(np.int64).reshape(c.G, 128)
        for j in range(i.shape[1] if n is None else n):
            ix = int(i[r, j])
            D = (a * c.signs[ix].astype(np.int64).reshape(c.G, 128)).sum(axis=1)
            b = 0.0 if c.bias is None else float(c.bias[ix])
            want = np.float32(binary_logit_f32(D, c.scales[ix], c.act_scale[m], b))
            got = np.float32(v[r, j])
            assert got.view(np.uint32) == want.view(np.uint32), (m, j, ix, got, want)


@pytest.mark.parametrize("M,G,C", [(1, 5, 0), (2, 40, 1024), (2, 3, 2048), (5, 13, 512),
                                   (8, 8, 0), (3, 32, 64)])
def test_logits_follow_the_documented_fp32_order(M, G, C):
    c = Case(M, 128 * G, 3001, seed=100 + G, with_bias=True)
    v, i = c.run(12, chunk_rows=C)
    assert_documented_fp32_order(c, v, i, list(range(M)))


@pytest.mark.parametrize("V", [3072 + 50, 1024 + 64, 4 * 1024, 2000])
@pytest.mark.parametrize("M", [1, 4, 6])
def test_ragged_last_chunk_one_wave_per_tile(M, V):
    """1,024-row chunks whose last chunk has from one tile up to all 16 (the
    waves without a tile of their own score none): the same bits as
    512-row chunks with two waves per tile."""
    c = Case(M, 2048, V, seed=V, with_bias=True)
    v0, i0, _ = c.check(40, chunk_rows=1024)
    v, i = c.run(40, chunk_rows=512)
    assert torch.equal(i, i0) and torch.equal(v.view(torch.int32), v0.view(torch.int32))
    assert_documented_fp32_order(c, v0, i0, list(range(M)), n=8)
