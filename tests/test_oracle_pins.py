"""Pins of the CPU oracle to facts outside itself (CPU only).

Each check targets a plausible mistake: a wrong tie rule or sign of zero in
the selection, a transposed operand, a dropped bias, a wrong group index or
scale in the binary projection, a wrong bit order or padding in the layout.
"""

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# selection
# --------------------------------------------------------------------------
def rank_by_counting(row):
    """rank(i) = #{j : x_j > x_i, or x_j == x_i and j < i} (pure Python)."""
    n = len(row)
    ranks = []
    for i in range(n):
        r = 0
        for j in range(n):
            if row[j] > row[i] or (row[j] == row[i] and j < i):
                r += 1
        ranks.append(r)
    return ranks


def test_topk_brute_force_all_small_patterns():
    """Every pattern over {-1, -0.0, +0.0, 1, 2}^V for V <= 5 and every k."""
    alphabet = [-1.0, -0.0, 0.0, 1.0, 2.0]
    for V in range(1, 6):
        for pattern in itertools.product(alphabet, repeat=V):
            row = np.array(pattern, dtype=np.float32)
            ranks = rank_by_counting(list(pattern))
            by_rank = [None] * V
            for i, r in enumerate(ranks):
                by_rank[r] = i
            for k in range(1, V + 1):
                vals, idx = oracle.topk_stable(row, k)
                assert list(idx) == by_rank[:k], (pattern, k)
                assert np.array_equal(vals.view(np.uint32), row[by_rank[:k]].view(np.uint32))


def test_topk_brute_force_random_with_ties():
    rng = np.random.default_rng(123)
    for trial in range(200):
        V = int(rng.integers(1, 40))
        row = rng.integers(-3, 4, size=V).astype(np.float64) * 0.5
        ranks = rank_by_counting(list(row))
        by_rank = sorted(range(V), key=lambda i: ranks[i])
        k = int(rng.integers(1, V + 1))
        _, idx = oracle.topk_stable(row, k)
        assert list(idx) == by_rank[:k]


def test_topk_golden_hand_worked():
    with open(os.path.join(GOLDEN, "topk_tiny.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        row = np.array([float(s) for s in case["row"]], dtype=np.float32)
        vals, idx = oracle.topk_stable(row, case["k"])
        assert list(idx) == case["indices"]
        # the value returned is that index's own bits (-0.0 stays -0.0)
        assert np.array_equal(vals.view(np.uint32), row[idx].view(np.uint32))


def test_k1_is_first_argmax():
    rng = np.random.default_rng(5)
    for _ in range(100):
        row = rng.integers(0, 5, size=int(rng.integers(1, 100))).astype(np.float32)
        _, idx = oracle.topk_stable(row, 1)
        assert idx[0] == int(np.argmax(row))  # np.argmax returns the first maximum


def test_all_equal_gives_first_k():
    row = np.full(1000, 0.25, dtype=np.float32)
    _, idx = oracle.topk_stable(row, 37)
    assert list(idx) == list(range(37))


def test_certificate_accepts_and_rejects():
    rng = np.random.default_rng(9)
    row = rng.integers(-5, 5, size=300).astype(np.float32)
    k = 40
    vals, idx = oracle.topk_stable(row, k)
    assert oracle.certify_topk(row, vals, idx, k)[0]
    # swapped pair
    i2 = idx.copy(); i2[[3, 4]] = i2[[4, 3]]
    assert not oracle.certify_topk(row, row[i2], i2, k)[0]
    # a left-out entry that beats the k-th
    i3 = idx.copy(); i3[-1] = int(np.argmin(row))
    assert not oracle.certify_topk(row, row[i3], i3, k)[0]
    # tie broken toward the higher index
    row4 = np.zeros(10, dtype=np.float32)
    assert not oracle.certify_topk(row4, row4[[1]], np.array([1]), 1)[0]
    assert oracle.certify_topk(row4, row4[[0]], np.array([0]), 1)[0]
    # wrong bits for a value (-0.0 reported as +0.0)
    row5 = np.array([-0.0, -1.0], dtype=np.float32)
    assert oracle.certify_topk(row5, np.array([-0.0], np.float32), np.array([0]), 1)[0]
    assert not oracle.certify_topk(row5, np.array([0.0], np.float32), np.array([0]), 1)[0]


# --------------------------------------------------------------------------
# dense projection
# --------------------------------------------------------------------------
def test_dense_integer_exact_and_non_square():
    """Small-integer inputs make float64 exact; compare with Python integers."""
    rng = np.random.default_rng(1)
    M, H, V = 3, 7, 11
    h = rng.integers(-9, 10, size=(M, H))
    w = rng.integers(-9, 10, size=(V, H))
    b = rng.integers(-9, 10, size=V)
    L = oracle.project_dense(h.astype(np.float32), w.astype(np.float32), b.astype(np.float32))
    assert L.shape == (M, V)
    for m in range(M):
        for v in range(V):
            exact = sum(int(h[m, j]) * int(w[v, j]) for j in range(H)) + int(b[v])
            assert L[m, v] == exact


def test_dense_one_hot_and_rank_one():
    rng = np.random.default_rng(2)
    V, H = 13, 16
    w = rng.standard_normal((V, H)).astype(np.float32)
    bias = rng.standard_normal(V).astype(np.float32)
    for j in (0, 5, H - 1):
        h = np.zeros((1, H), dtype=np.float32); h[0, j] = 1.0
        L = oracle.project_dense(h, w, bias)
        assert np.array_equal(L[0], w[:, j].astype(np.float64) + bias.astype(np.float64))
    # rank one: W[v, j] = u_v * z_j  =>  L[m, v] = u_v * (h_m . z), powers of two keep it exact
    u = 2.0 ** rng.integers(-3, 4, size=V)
    z = 2.0 ** rng.integers(-3, 4, size=H)
    W = np.outer(u, z).astype(np.float32)
    h = (2.0 ** rng.integers(-3, 4, size=(2, H))).astype(np.float32)
    L = oracle.project_dense(h, W)
    for m in range(2):
        hz = sum(Fraction(float(h[m, j])) * Fraction(float(z[j])) for j in range(H))
        for v in range(V):
            assert Fraction(L[m, v]) == Fraction(float(u[v])) * hz


def test_bf16_widening():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x7F80, 0x4049, 0x0001], dtype=np.uint16)
    f = oracle.bf16_bits_to_f32(bits)
    assert f[0] == 1.0 and f[1] == -1.0 and f[2] == 0.0 and np.signbit(f[3]) and f[3] == 0.0
    assert np.isinf(f[4])
    assert f[5] == np.float32(3.140625)          # 0x4049 = 1.5703125 * 2
    assert f[6] == np.float32(2.0 ** -133)       # smallest bf16 subnormal


# --------------------------------------------------------------------------
# binary projection
# --------------------------------------------------------------------------
def _tiny_binary(rng, M, V, H):
    act_q = rng.integers(-128, 128, size=(M, H)).astype(np.int8)
    act_scale = (rng.random(M).astype(np.float32) + np.float32(0.01))
    signs = np.where(rng.random((V, H)) < 0.5, 1, -1).astype(np.int8)
    scales = rng.random((V, H // 128)).astype(np.float32)
    bias = rng.standard_normal(V).astype(np.float32)
    return act_q, act_scale, signs, scales, bias


def test_binary_one_hot_hits_the_right_group():
    """act_q = a * e_j: L_v = act_scale * a * sign[v, j] * scale[v, j // 128] + bias_v."""
    rng = np.random.default_rng(3)
    V, H = 9, 512
    _, _, signs, scales, bias = _tiny_binary(rng, 1, V, H)
    for j, a in ((0, 127), (127, -128), (128, 5), (300, -77), (511, 1)):
        act_q = np.zeros((1, H), dtype=np.int8); act_q[0, j] = a
        act_scale = np.array([0.375], dtype=np.float32)
        L = oracle.project_binary(act_q, act_scale, signs, scales, bias)
        for v in range(V):
            expect = (Fraction(0.375) * a * int(signs[v, j]) * Fraction(float(scales[v, j // 128]))
                      + Fraction(float(bias[v])))
            assert abs(Fraction(L[0, v]) - expect) <= abs(expect) * Fraction(1, 2 ** 50)


def test_binary_exact_rationals():
    """float64 result within 2^-45 relative of the exact rational value."""
    rng = np.random.default_rng(4)
    M, V, H = 2, 5, 256
    act_q, act_scale, signs, scales, bias = _tiny_binary(rng, M, V, H)
    L = oracle.project_binary(act_q, act_scale, signs, scales, bias)
    for m in range(M):
        for v in range(V):
            acc = Fraction(0)
            for j in range(H):
                acc += int(act_q[m, j]) * int(signs[v, j]) * Fraction(float(scales[v, j // 128]))
            exact = acc * Fraction(float(act_scale[m])) + Fraction(float(bias[v]))
            mag = sum(abs(int(act_q[m, j])) * Fraction(float(scales[v, j // 128])) for j in range(H))
            tol = (mag * Fraction(float(act_scale[m])) + abs(Fraction(float(bias[v])))) * Fraction(1, 2 ** 45)
            assert abs(Fraction(L[m, v]) - exact) <= tol


def test_binary_closed_forms_and_symmetry():
    rng = np.random.default_rng(6)
    V, H = 4, 384
    scales = rng.random((V, 3)).astype(np.float32)
    # all +1 signs and a constant activation a: L = act_scale * a * 128 * sum_g scale_g
    signs = np.ones((V, H), dtype=np.int8)
    act_q = np.full((1, H), 3, dtype=np.int8)
    L = oracle.project_binary(act_q, np.array([0.5], np.float32), signs, scales)
    for v in range(V):
        expect = 0.5 * 3 * 128 * sum(float(s) for s in scales[v])
        assert math.isclose(L[0, v], expect, rel_tol=1e-14)
    # flipping every sign negates the bias-free logit exactly
    act_q, act_scale, signs, scales, _ = _tiny_binary(rng, 2, V, H)
    L1 = oracle.project_binary(act_q, act_scale, signs, scales)
    L2 = oracle.project_binary(act_q, act_scale, (-signs).astype(np.int8), scales)
    assert np.array_equal(L1, -L2)
    # bias enters once, additively
    bias = rng.standard_normal(V).astype(np.float32)
    L3 = oracle.project_binary(act_q, act_scale, signs, scales, bias)
    assert np.allclose(L3 - L1, bias.astype(np.float64)[None, :], rtol=0, atol=1e-12)


def test_binary_equals_dense_on_dequantized_weights():
    """The binary projection is the dense one on x = act_q*act_scale, W = sign*scale."""
    rng = np.random.default_rng(7)
    M, V, H = 3, 17, 256
    act_q, act_scale, signs, scales, bias = _tiny_binary(rng, M, V, H)
    x = act_q.astype(np.float64) * act_scale.astype(np.float64)[:, None]
    W = np.empty((V, H))
    for v in range(V):
        for j in range(H):
            W[v, j] = float(signs[v, j]) * float(scales[v, j // 128])
    Lb = oracle.project_binary(act_q, act_scale, signs, scales, bias)
    Ld = oracle.project_dense(x, W, bias)
    assert np.allclose(Lb, Ld, rtol=1e-13, atol=0)


# --------------------------------------------------------------------------
# packing and layout
# --------------------------------------------------------------------------
def test_pack_recovers_known_signs_and_scales():
    rng = np.random.default_rng(8)
    V, H = 70, 384
    signs = np.where(rng.random((V, H)) < 0.5, 1, -1).astype(np.int8)
    scales = rng.random((V, H // 128)).astype(np.float32) + np.float32(0.5)
    W = (signs.astype(np.float32) * np.repeat(scales, 128, axis=1)).astype(np.float32)
    s2, sc2 = oracle.pack_logical(W)
    assert np.array_equal(s2, signs)
    assert np.array_equal(sc2.view(np.uint32), scales.view(np.uint32))  # 128 equal values: exact mean


def test_pack_zero_sign_and_mean():
    W = np.zeros((2, 128), dtype=np.float32)
    W[0, :] = -0.0
    W[1, :] = np.arange(1, 129, dtype=np.float32)
    W[1, 0] = -1.0
    s, sc = oracle.pack_logical(W)
    assert np.all(s[0] == 1)                   # -0.0 >= 0 packs as +1
    assert s[1, 0] == -1 and np.all(s[1, 1:] == 1)
    assert sc[0, 0] == 0.0 and sc[1, 0] == np.float32(64.5)   # mean of 1..128


def _golden_head(g):
    V, H = g["V"], g["H"]
    W = np.full((V, H), -1.0, dtype=np.float32)
    j = np.arange(H)
    W[0] = 1.0
    W[1] = np.where(j % 2 == 0, 2.0, -2.0)
    W[63] = np.where(j < 32, 0.5, -0.5)
    W[64] = np.where(j < 128, -0.0, -3.0)
    W[64, 165] = 3.0
    return W


def test_layout_golden_hand_derived():
    with open(os.path.join(GOLDEN, "layout_v1_tiny.json")) as f:
        g = json.load(f)
    W = _golden_head(g)
    signs, scales = oracle.pack_logical(W)
    wq, ws = oracle.pack_layout_bytes(signs, scales)
    assert wq.shape == (g["total_words"],) and ws.shape == (g["total_scales"],)
    wq_b, ws_b = oracle.packed_sizes(g["V"], g["H"])
    assert wq_b == 4 * g["total_words"] and ws_b == 4 * g["total_scales"]
    expect = np.zeros_like(wq)
    for k, v in g["expected_words"].items():
        expect[int(k)] = int(v, 16)
    assert np.array_equal(wq, expect)
    expect_s = np.zeros_like(ws)
    for r in range(2, 63):
        expect_s[4 * r] = 1.0
        expect_s[4 * r + 1] = 1.0
    for k, v in g["expected_scales"].items():
        expect_s[int(k)] = v
    assert np.array_equal(ws, expect_s)
    # the reader inverts the writer
    s2, sc2 = oracle.unpack_layout_bytes(wq, ws, g["V"], g["H"])
    assert np.array_equal(s2, signs) and np.array_equal(sc2, scales)


def test_layout_round_trip_random_ragged():
    rng = np.random.default_rng(10)
    for V, H in ((1, 128), (63, 128), (65, 640), (130, 256)):
        signs = np.where(rng.random((V, H)) < 0.5, 1, -1).astype(np.int8)
        scales = rng.random((V, H // 128)).astype(np.float32)
        wq, ws = oracle.pack_layout_bytes(signs, scales)
        wqb, wsb = oracle.packed_sizes(V, H)
        assert wq.nbytes == wqb and ws.nbytes == wsb
        s2, sc2 = oracle.unpack_layout_bytes(wq, ws, V, H)
        assert np.array_equal(s2, signs) and np.array_equal(sc2, scales)


# --------------------------------------------------------------------------
# input generators (not the method, but both sides depend on them)
# --------------------------------------------------------------------------
def test_generators_deterministic_and_thread_independent():
    a = synthetic.normal_rows(20000, 8, seed=3, stream=1, threads=1)
    b = synthetic.normal_rows(20000, 8, seed=3, stream=1, threads=4)
    assert np.array_equal(a, b)
    q, s = synthetic.quantize_rows_int8(np.array([[0.0, 1.5, -2.0, 0.25]], np.float32))
    assert s[0] == np.float32(2.0 / 127.0)
    assert list(q[0]) == [0, 95, -127, 16]  # 95.25 -> 95, 15.875 -> 16
    q0, s0 = synthetic.quantize_rows_int8(np.zeros((1, 4), np.float32))
    assert s0[0] == 1.0 and not q0.any()
    bits = synthetic.f32_to_bf16_bits(np.array([1.0, 1.00390625, 1.01171875, -2.5], np.float32))
    # 1 + 2^-8 is halfway between bf16 neighbours 1 and 1 + 2^-7: ties to even -> 1.0
    assert list(bits) == [0x3F80, 0x3F80, 0x3F82, 0xC020]


# ---------------------------------------------------------------------------
# log-sum-exp (Selective Log Softmax page: log-probability = logit - lse)
# ---------------------------------------------------------------------------
def test_logsumexp_closed_forms():
    # V equal logits c: lse = c + log(V); one logit: lse = that logit
    for V in (1, 2, 7, 1000, 248320):
        for c in (0.0, -3.5, 12.25):
            assert math.isclose(oracle.logsumexp_row(np.full(V, c)), c + math.log(V),
                                rel_tol=0, abs_tol=1e-12 * max(1.0, abs(c) + math.log(V)))
    assert oracle.logsumexp_row(np.array([-7.25])) == -7.25
    # two entries a, b: lse = max + log1p(exp(-|a - b|))
    for a, b in ((1.0, 2.0), (-30.0, 5.0), (0.5, 0.5)):
        want = max(a, b) + math.log1p(math.exp(-abs(a - b)))
        assert math.isclose(oracle.logsumexp_row(np.array([a, b])), want, rel_tol=1e-15, abs_tol=1e-15)


def test_logsumexp_brute_force_and_shift():
    rng = np.random.default_rng(11)
    x = rng.normal(0.0, 2.0, size=513)
    # the plain log of the plain sum (no overflow at this scale), summed exactly
    brute = math.log(math.fsum(math.exp(v) for v in x))
    assert math.isclose(oracle.logsumexp_row(x), brute, rel_tol=1e-14, abs_tol=1e-14)
    # shift invariance far outside the range exp can represent unshifted
    for c in (-1000.0, 700.0, 1e4):
        assert math.isclose(oracle.logsumexp_row(x + c), brute + c, rel_tol=1e-13, abs_tol=1e-10)


def test_logsumexp_matches_an_independent_routine_and_infinities():
    scipy_special = pytest.importorskip("scipy.special")
    rng = np.random.default_rng(12)
    L = rng.normal(0.0, 3.0, size=(4, 2049)).astype(np.float32)
    got = oracle.logsumexp_rows(L)
    want = scipy_special.logsumexp(L.astype(np.float64), axis=1)
    assert np.allclose(got, want, rtol=1e-14, atol=1e-14)
    row = np.array([0.0, -np.inf, 3.0])
    assert math.isclose(oracle.logsumexp_row(row), 3.0 + math.log1p(math.exp(-3.0)), rel_tol=1e-15)
    assert oracle.logsumexp_row(np.array([1.0, np.inf, -np.inf])) == np.inf
    assert oracle.logsumexp_row(np.full(5, -np.inf)) == -np.inf


# ---------------------------------------------------------------------------
# grammar bitmask (logits-processor page: bit 1 = allowed, disallowed -> -inf)
# ---------------------------------------------------------------------------
def test_mask_hand_worked_words():
    # word 0 = 0b101 allows entries 0 and 2; word 1 bit 0 allows entry 32; bit 31
    # of word 0 (a negative int32) allows entry 31; bits past V are ignored
    V = 34
    bm = np.array([[0b101 | -2**31, 0b1 | 0b100]], dtype=np.int32)
    allowed = oracle.allowed_bool(bm, V)
    assert sorted(np.flatnonzero(allowed[0]).tolist()) == [0, 2, 31, 32]
    L = np.arange(V, dtype=np.float32)[None, :]
    out = oracle.apply_allowed(L, bm)
    assert out[0, 2] == 2.0 and out[0, 32] == 32.0 and out[0, 1] == -np.inf and out[0, 33] == -np.inf
    assert L[0, 1] == 1.0  # the input is not modified


def test_mask_all_and_none_and_independent_packing():
    rng = np.random.default_rng(21)
    M, V = 3, 1000
    L = rng.normal(size=(M, V)).astype(np.float32)
    W = (V + 31) // 32
    assert np.array_equal(oracle.apply_allowed(L, np.full((M, W), -1, dtype=np.int32)), L)
    assert np.all(oracle.apply_allowed(L, np.zeros((M, W), dtype=np.int32)) == -np.inf)
    want = rng.random((M, V)) < 0.3
    # NumPy's own little-endian bit packing, read as little-endian int32 words
    padded = np.zeros((M, W * 32), dtype=bool)
    padded[:, :V] = want
    bm = np.packbits(padded, axis=1, bitorder="little").view("<i4")
    assert np.array_equal(oracle.allowed_bool(bm, V), want)
    assert np.array_equal(oracle.apply_allowed(L, bm), np.where(want, L, -np.inf).astype(np.float32))


def test_topk_stable_rows_brute_force_and_dtype():
    """Each row's (values, indices) equal the brute-force ranking of that row,
    and the values keep the input's dtype and bits."""
    rng = np.random.default_rng(22)
    for dtype in (np.float32, np.float64):
        L = np.floor(rng.normal(size=(5, 40)) * 3).astype(dtype)
        L[1, 3] = -0.0
        L[2, :] = 1.0
        for k in (1, 7, 40):
            vals, idx = oracle.topk_stable_rows(L, k)
            assert vals.dtype == dtype and idx.dtype == np.int64
            assert vals.shape == (5, k) and idx.shape == (5, k)
            for m in range(5):
                ranks = rank_by_counting(L[m].tolist())
                want = sorted(range(40), key=lambda i: ranks[i])[:k]
                assert idx[m].tolist() == want
                assert np.array_equal(vals[m].view(np.uint8), L[m, want].view(np.uint8))


# ---------------------------------------------------------------------------
# sampling over the survivors (logits-processor page, sections "API" and
# "Method": temperature, top-k / top-p / min-p keep set, Gumbel-max draw
# keyed by (seed, row, offset))
# ---------------------------------------------------------------------------
def test_philox_known_answer_vectors():
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        ctr = [int(x, 16) for x in case["counter"]]
        key = [int(x, 16) for x in case["key"]]
        want = tuple(int(x, 16) for x in case["out"])
        assert oracle.philox4x32_10(ctr, key) == want


def test_uniform_and_gumbel_closed_forms():
    # u = (x >> 9 + 1/2) * 2^-23: ends of the range, and every value fits fp32
    assert oracle.uniform_from_word(0) == 2.0 ** -24
    assert oracle.uniform_from_word(0xFFFFFFFF) == 1.0 - 2.0 ** -24
    assert oracle.uniform_from_word(1 << 31) == 0.5 + 2.0 ** -24
    assert oracle.uniform_from_word(511) == oracle.uniform_from_word(0)  # low 9 bits dropped
    for x in (0, 12345, 1 << 31, 0xFFFFFFFF, 0xDEADBEEF):
        u = oracle.uniform_from_word(x)
        assert float(np.float32(u)) == u and 0.0 < u < 1.0
    # the Gumbel inverse CDF: F(x) = exp(-exp(-x)), so gumbel(F(x)) = x
    for x in (-2.0, 0.0, 0.5, 3.0, 10.0):
        assert math.isclose(oracle.gumbel(math.exp(-math.exp(-x))), x, rel_tol=1e-12, abs_tol=1e-12)
    # larger u, larger noise
    us = [oracle.uniform_from_word(x) for x in (0, 1 << 20, 1 << 30, 3 << 30, 0xFFFFFFFF)]
    gs = [oracle.gumbel(u) for u in us]
    assert all(a < b for a, b in zip(gs, gs[1:]))


def test_draw_keying():
    """The uniform depends on every part of the key (seed, row, offset incl.
    its high word, vocabulary entry) and nothing else."""
    base = oracle.draw_uniform(7, 2, 5, 1000)
    assert oracle.draw_uniform(7, 2, 5, 1000) == base
    others = [oracle.draw_uniform(8, 2, 5, 1000), oracle.draw_uniform(7, 3, 5, 1000),
              oracle.draw_uniform(7, 2, 6, 1000), oracle.draw_uniform(7, 2, 5, 1001),
              oracle.draw_uniform(7, 2, 5 + (1 << 32), 1000), oracle.draw_uniform(7 + (1 << 32), 2, 5, 1000)]
    assert all(u != base for u in others)
    # the word it uses is the first output of the generator at that counter and key
    x = oracle.philox4x32_10((1000, 2, 5, 0), (7, 0))[0]
    assert base == oracle.uniform_from_word(x)


def test_keep_count_hand_worked():
    # probabilities 1/2, 1/4, 1/8, 1/8 over the whole vocabulary (lse = 0)
    z = np.log(np.array([0.5, 0.25, 0.125, 0.125]))
    kc = oracle.keep_count
    assert kc(z, 0.0, 0, 1.0, 0.0) == 4          # every filter off
    assert kc(z, 0.0, 3, 1.0, 0.0) == 3          # top-k
    assert kc(z, 0.0, 10, 1.0, 0.0) == 4         # top_k beyond k: k
    assert kc(z, 0.0, 0, 0.49, 0.0) == 1         # mass before position 1 is 1/2
    assert kc(z, 0.0, 0, 0.74, 0.0) == 2         # 3/4 before position 2
    assert kc(z, 0.0, 0, 0.76, 0.0) == 3         # 7/8 before position 3
    assert kc(z, 0.0, 0, 0.9, 0.0) == 4
    assert kc(z, 0.0, 0, 1.0, 0.3) == 2          # ratios 1, 1/2, 1/4, 1/4
    assert kc(z, 0.0, 0, 1.0, 0.2) == 4
    assert kc(z, 0.0, 3, 0.9, 0.2) == 3          # the intersection is the shortest prefix
    assert kc(z, 0.0, 0, 0.76, 0.3) == 2
    assert kc(np.array([0.0, -np.inf, -np.inf]), 0.0, 0, 1.0, 0.0) == 1
    # a normalizer over a larger vocabulary scales the probabilities down
    # probabilities 1/4, 1/8, 1/16, 1/16: masses before positions 1..3 are
    # 1/4, 3/8, 7/16
    assert kc(z, math.log(2.0), 0, 0.4, 0.0) == 3
    assert kc(z, math.log(2.0), 0, 0.45, 0.0) == 4


def _cutoff_keep(p_full, k, top_k, top_p, min_p):
    """The filters as one probability cutoff over the whole vocabulary (the
    logits-processor page's formulation), for distinct probabilities: the
    number of tokens whose probability is at least every filter's cutoff,
    then limited to the k survivors."""
    p = np.sort(np.asarray(p_full))[::-1]
    cuts = [0.0]
    if top_k > 0:
        cuts.append(p[min(top_k, len(p)) - 1])
    if top_p < 1.0:
        csum = np.cumsum(p)
        n = int(np.searchsorted(csum, top_p, side="left")) + 1  # first n with mass >= top_p
        cuts.append(p[min(n, len(p)) - 1])
    if min_p > 0.0:
        cuts.append(min_p * p[0])
    return min(int(np.sum(p >= max(cuts))), k)


def test_keep_count_equals_single_cutoff():
    rng = np.random.default_rng(23)
    for trial in range(300):
        V = int(rng.integers(2, 40))
        L = rng.normal(0.0, 2.0, size=V)
        T = float(rng.choice([0.5, 1.0, 1.7]))
        k = int(rng.integers(1, V + 1))
        top_k = int(rng.choice([0, 1, 3, 8, 100]))
        top_p = float(rng.choice([1.0, 0.3, 0.8, 0.95]))
        min_p = float(rng.choice([0.0, 0.05, 0.3]))
        zf = L / T
        lse = oracle.logsumexp_row(zf)
        p_full = np.exp(zf - lse)
        vals, idx = oracle.topk_stable(L, k)
        got = oracle.keep_count(vals / T, lse, top_k, top_p, min_p)
        want = _cutoff_keep(p_full, k, top_k, top_p, min_p)
        # the cumulative sums are only float64-exact: skip draws within rounding of a cut
        csum = np.cumsum(np.sort(p_full)[::-1])
        if np.min(np.abs(csum - top_p)) < 1e-12 or np.min(np.abs(p_full / p_full.max() - min_p)) < 1e-12:
            continue
        assert got == max(1, want), (trial, got, want)


def test_sample_greedy_cases():
    rng = np.random.default_rng(24)
    L = rng.normal(size=(3, 50))
    L[1, 7] = L[1, 30] = L[1].max() + 1.0  # tie for the maximum: lower index
    first_max = [int(np.argmax(L[m])) for m in range(3)]
    for kw in ({"temperature": 0.0}, {"temperature": -1.0}, {"top_k": 1}, {"top_p": 0.0}):
        for k in (1, 5, 50):
            args = dict(temperature=0.8, top_k=0, top_p=1.0, min_p=0.0, seed=3, offset=9)
            args.update(kw)
            tokens, kept = oracle.sample_rows(L, k, **args)
            assert tokens.tolist() == first_max and kept.tolist() == [1, 1, 1]
    # min_p = 1 keeps exactly the entries equal to the maximum (both tied ones in row 1)
    tokens, kept = oracle.sample_rows(L, 50, temperature=0.8, min_p=1.0, seed=3, offset=9)
    assert kept.tolist() == [1, 2, 1] and tokens[1] in (7, 30)
    assert tokens[0] == first_max[0] and tokens[2] == first_max[2]
    # k = 1 whatever the parameters
    tokens, kept = oracle.sample_rows(L, 1, temperature=2.0, top_p=1.0, seed=1, offset=2)
    assert tokens.tolist() == first_max and kept.tolist() == [1, 1, 1]
    # an +inf logit wins outright; an all -inf row returns its first index
    Li = np.array([[0.0, np.inf, 1.0, np.inf], [-np.inf] * 4])
    tokens, kept = oracle.sample_rows(Li, 3, temperature=1.0, seed=0, offset=0)
    assert tokens.tolist() == [1, 0] and kept.tolist() == [1, 1]


def test_gumbel_max_matches_the_filtered_softmax():
    """20,000 draws (offsets 0..19,999) land in the keep set only, with the
    frequencies of the renormalized softmax over it (chi-square, p < 1e-6
    would fail): a wrong sign or scale of the noise, or of the temperature,
    fails this."""
    scipy_stats = pytest.importorskip("scipy.stats")
    L = np.array([[2.0, 1.2, 1.0, 0.3, -0.5, -1.0, -3.0, 0.9]])
    T, top_p, min_p, k = 0.8, 0.9, 0.05, 6
    r = oracle.sample_row(L[0], k, T, 0, top_p, min_p, seed=11, row=0, offset=0)
    n = r["kept"]
    keep_idx = r["indices"][:n].tolist()
    assert 2 <= n < k  # the filters bite in this case
    w = np.exp(r["z"][:n] - r["z"][0])
    expect = w / w.sum()
    draws = 20000
    counts = dict.fromkeys(keep_idx, 0)
    for off in range(draws):
        tok = oracle.sample_row(L[0], k, T, 0, top_p, min_p, seed=11, row=0, offset=off)["token"]
        assert tok in counts
        counts[tok] += 1
    obs = np.array([counts[i] for i in keep_idx], dtype=np.float64)
    stat = float(np.sum((obs - draws * expect) ** 2 / (draws * expect)))
    assert stat < scipy_stats.chi2.ppf(1.0 - 1e-6, n - 1), (stat, obs, draws * expect)


def test_sample_rows_per_row_parameters():
    rng = np.random.default_rng(25)
    M, V, k = 4, 300, 40
    L = rng.normal(size=(M, V))
    T = np.array([0.0, 0.5, 1.0, 2.0])
    tk = np.array([0, 5, 40, 3])
    tp = np.array([1.0, 0.9, 0.5, 1.0])
    mp = np.array([0.0, 0.0, 0.1, 0.5])
    tokens, kept = oracle.sample_rows(L, k, T, tk, tp, mp, seed=5, offset=77)
    for m in range(M):
        r = oracle.sample_row(L[m], k, T[m], tk[m], tp[m], mp[m], seed=5, row=m, offset=77)
        assert tokens[m] == r["token"] and kept[m] == r["kept"]
    assert kept[0] == 1 and kept[3] <= 3
    # the row is part of the key: equal rows draw differently at some offset
    L2 = np.repeat(L[:1], 2, axis=0)
    diff = 0
    for off in range(20):
        t2, _ = oracle.sample_rows(L2, k, 1.0, 0, 1.0, 0.0, seed=5, offset=off)
        diff += int(t2[0] != t2[1])
    assert diff > 0
