"""Selection stage on fp32 logits: bit-exact against the oracle (GPU).

The chunk select and merge kernels are the ones the fused paths use; here
they are fed from logits in memory so every result can be compared bit for
bit (lm-head-topk page, section "Method": per-chunk top-k and a merge; ties to
the lower index; section "Correctness": k = 1 is the argmax, ragged last
chunk, all winners in one chunk, repeated calls identical).
"""

import itertools

import numpy as np
import pytest
import torch

import oracle
import synthetic
from parity import assert_select_exact

pytestmark = pytest.mark.gpu

import lm_head_projection_amd as lt  # noqa: E402


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def run_select(logits_np, k, chunk_rows=0):
    v, i = lt.topk_logits(dev(logits_np), k, chunk_rows=chunk_rows)
    torch.cuda.synchronize()
    return v.cpu().numpy(), i.cpu().numpy()


def test_tiny_brute_force_patterns():
    alphabet = np.array([-1.0, -0.0, 0.0, 1.0, 2.0], dtype=np.float32)
    for V in range(1, 5):
        pats = np.array(list(itertools.product(range(5), repeat=V)))
        # batch the patterns as rows of M <= 8
        for s in range(0, len(pats), 8):
            rows = alphabet[pats[s:s + 8]]
            for k in range(1, V + 1):
                v, i = run_select(rows, k)
                assert_select_exact(rows, v, i, k)


@pytest.mark.parametrize("k", [1, 7, 50, 64, 1024, 2048])
@pytest.mark.parametrize("chunk_rows", [0, 64, 192, 256, 1024, 2048])
def test_random_rows_all_chunk_sizes(k, chunk_rows):
    x = synthetic.random_logits(3, 50000, seed=11)
    v, i = run_select(x, k, chunk_rows)
    assert_select_exact(x, v, i, k)


@pytest.mark.parametrize("ties", [3, 20, 200])
@pytest.mark.parametrize("k", [1, 50, 999])
def test_heavy_ties_and_signed_zeros(ties, k):
    x = synthetic.random_logits(4, 32001, seed=ties, ties=ties, signed_zeros=True)
    v, i = run_select(x, k)
    assert_select_exact(x, v, i, k)
    v2, i2 = run_select(x, k, chunk_rows=512)
    assert np.array_equal(i, i2) and np.array_equal(v.view(np.uint32), v2.view(np.uint32))


def test_infinities_and_all_equal():
    x = synthetic.random_logits(4, 5000, seed=3)
    x[0, ::97] = np.inf
    x[1, ::13] = -np.inf
    x[2, :] = np.float32(0.5)
    x[3, :] = -np.inf
    x[3, 4321] = np.float32(-1e30)
    for k in (1, 10, 100):
        v, i = run_select(x, k)
        assert_select_exact(x, v, i, k)


def test_k_equals_v_full_sort():
    for V in (1, 63, 64, 65, 1000, 2048):
        x = synthetic.random_logits(2, V, seed=V, ties=10)
        v, i = run_select(x, V)
        assert_select_exact(x, v, i, V)


def test_all_winners_in_one_chunk_and_ragged_tail():
    V, k = 32001, 50
    for C in (1024, 2048):
        x = synthetic.random_logits(2, V, seed=7)
        # row 0: every winner inside chunk 7; row 1: every winner in the ragged last chunk
        x[0, 7 * C: 7 * C + 50] += np.float32(100.0)
        last = (V - 1) // C * C
        x[1, last: last + 50] += np.float32(100.0)
        v, i = run_select(x, k, C)
        assert_select_exact(x, v, i, k)
        assert set(i[0]) == set(range(7 * C, 7 * C + 50))
        assert set(i[1]) == set(range(last, last + 50))


def test_k1_is_argmax_and_strided_rows():
    base = synthetic.random_logits(8, 40000, seed=5, ties=50)
    t = dev(base)
    wide = torch.zeros((8, 40960), dtype=torch.float32, device="cuda")
    wide[:, :40000] = t
    view = wide[:, :40000]  # row stride 40960 > V
    v, i = lt.topk_logits(view, 1)
    torch.cuda.synchronize()
    assert np.array_equal(i.cpu().numpy()[:, 0], np.argmax(base, axis=1))
    v, i = lt.topk_logits(view, 300)
    torch.cuda.synchronize()
    assert_select_exact(base, v.cpu().numpy(), i.cpu().numpy(), 300)


@pytest.mark.parametrize("M,k", [(1, 50), (8, 50), (8, 1024), (2, 2048)])
def test_flagship_vocabulary(M, k):
    x = synthetic.random_logits(M, 248320, seed=M * 1000 + k)
    v, i = run_select(x, k)
    assert_select_exact(x, v, i, k)


def test_repeat_bitwise_identical():
    x = synthetic.random_logits(8, 248320, seed=99, ties=1000)
    t = dev(x)
    v0, i0 = lt.topk_logits(t, 50)
    for _ in range(10):
        v, i = lt.topk_logits(t, 50)
        assert torch.equal(i, i0) and torch.equal(v.view(torch.int32), v0.view(torch.int32))
    assert_select_exact(x, v0.cpu().numpy(), i0.cpu().numpy(), 50)


@pytest.mark.parametrize("copies", [1, 2, 3, 50])
def test_equal_chunk_maxima_bound_and_fallback(copies):
    # Every 1024-row chunk of a 248,320-entry row peaks at the same value, in
    # `copies` places: the k-th largest chunk maximum then equals the k-th
    # largest logit, and 243 * copies candidates tie with it (fewer or more
    # than the merge's survivor buffer holds), so the answer is the k lowest
    # indices holding the peak.
    V, C, k = 248320, 1024, 50
    x = synthetic.random_logits(2, V, seed=copies)
    x = np.minimum(x, np.float32(3.0))
    for c in range(0, V, C):
        for j in range(copies):
            x[:, c + 10 * j + 5] = np.float32(4.0)  # inside the 512-row last chunk too
    x[1] = -x[1]  # row 1: peaks become minima, its own random maxima decide
    v, i = run_select(x, k, C)
    assert_select_exact(x, v, i, k)
    peaks = np.flatnonzero(x[0] == np.float32(4.0))
    assert np.array_equal(i[0], peaks[:k])


def _hip_runtime():
    import ctypes
    with open("/proc/self/maps") as f:
        path = next(line.split()[-1] for line in f if "libamdhip64" in line)
    hip = ctypes.CDLL(path)
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                        ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return hip


def test_score_events_time_the_scoring_kernel():
    # the options' event pair records the scoring kernel's own start and end;
    # results are unchanged
    import ctypes
    torch.zeros(1, device="cuda")
    hip = _hip_runtime()
    ev = [ctypes.c_void_p(), ctypes.c_void_p()]
    for e in ev:
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
    x = synthetic.random_logits(2, 248320, seed=4)
    t = dev(x)
    v0, i0 = lt.topk_logits(t, 50)
    v1, i1 = lt.topk_logits(t, 50, score_events=(ev[0], ev[1]))
    torch.cuda.synchronize()
    ms = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(ms), ev[0], ev[1]) == 0
    assert 0.0 < ms.value < 100.0
    assert torch.equal(i0, i1) and torch.equal(v0.view(torch.int32), v1.view(torch.int32))
    for e in ev:
        hip.hipEventDestroy(e)


@pytest.mark.parametrize("layout", ["one_chunk", "last_chunk", "five_per_chunk", "k_above_heads"])
def test_merge_reads_whole_chunks_when_heads_may_not_suffice(layout):
    # 243 chunks of 1024 rows: the merge bounds the survivors by the chunk
    # maxima and reads only each chunk's four best candidates, except for
    # chunks whose fourth best passes the bound; these layouts force that.
    V, C = 248320, 1024
    k = 50
    x = synthetic.random_logits(1, V, seed=21)
    if layout == "one_chunk":
        x[0, 7 * C + 3: 7 * C + 3 + 50 * 19: 19] += np.float32(100.0)
    elif layout == "last_chunk":
        last = (V - 1) // C * C
        x[0, last: last + 50] += np.float32(100.0)
    elif layout == "five_per_chunk":
        for c in range(0, 30 * C, 3 * C):  # 10 chunks, 5 winners each
            x[0, c + 100: c + 105] += np.float32(50.0)
    else:
        k = 200  # k-th best far below the chunk maxima: many chunks pass
    v, i = run_select(x, k, C)
    assert_select_exact(x, v, i, k)


@pytest.mark.parametrize("V,k", [(3092, 50), (3172, 50), (3172, 64), (3172, 1), (4096 + 300, 64),
                                 (1024 * 5 + 64, 8)])
def test_small_k_chunk_path_ragged_tails(V, k):
    # chunks of 1024 rows with k <= 64 take the per-wave-tops threshold; the
    # last chunk here holds fewer rows than k, or few rows in few waves
    x = synthetic.random_logits(3, V, seed=V + k, ties=0)
    v, i = run_select(x, k, 1024)
    assert_select_exact(x, v, i, k)
    v2, i2 = run_select(x, k, 2048)
    assert np.array_equal(i, i2)


@pytest.mark.parametrize("V,k,C", [(4096, 50, 512), (2048, 256, 512), (2560, 205, 512), (4096, 200, 256),
                                   (20000, 250, 1024), (4096, 512, 512), (20000, 300, 1024),
                                   (9000, 300, 1024), (16384, 1024, 1024)])
def test_full_merge_slot_forms(V, k, C):
    # fewer chunks than k: the merge selects over all n_chunks * k
    # candidates, with 1, 4 or the full count of slots per thread depending
    # on how many there are (here from 400 to 16,384, with the boundaries
    # 1,024 and 4,096 and one above each).  Up to k = 256 the chunk launch's
    # last workgroup merges and ranks them; above, a merge launch selects and
    # radix-sorts them.
    x = synthetic.random_logits(2, V, seed=V + k + C, ties=5)
    v, i = run_select(x, k, C)
    assert_select_exact(x, v, i, k)


@pytest.mark.parametrize("V", [40000, 80000])
def test_two_level_merge_with_key_histogram(V):
    # k = 1,024 over all rows of 1,024-row chunks: the merge counts the keys
    # first, its first level keeps the keys in or above the bin of the k-th
    # largest, and the last level gathers what the segments kept (row 0)
    # unless that is more than 4 slots per thread (row 1: all logits equal,
    # every segment keeps k, 5 segments at V = 80,000) and reads the padded
    # segments instead
    x = synthetic.random_logits(3, V, seed=V, ties=3)
    x[1, :] = np.float32(0.25)
    x[2, : V // 2] = np.float32(-1.0)  # half of row 2 equal, below the rest
    v, i = run_select(x, 1024, 1024)
    assert_select_exact(x, v, i, 1024)
    assert np.array_equal(i[1], np.arange(1024))


def test_fused_merge_counter_is_left_zero_and_workspace_is_shared():
    # A call whose candidates fit one chunk workgroup merges in the last
    # workgroup to finish, counted on the workspace's first word, which every
    # call leaves at zero.  One workspace serves fused (k = 50, 7) and
    # two-level (k = 1024) calls in any order, and repeated calls.
    V = 248320
    x = synthetic.random_logits(8, V, seed=77, ties=100)
    t = dev(x)
    ws = lt.new_workspace(8, V, 1024, device="cuda")
    assert lt.workspace_bytes(8, V, 50) <= ws.numel()
    for k in (50, 1024, 7, 50, 1024, 50):
        v, i = lt.topk_logits(t, k, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws[:65792].count_nonzero()) == 0, f"counter / key histograms not zero after k={k}"
        assert_select_exact(x, v.cpu().numpy(), i.cpu().numpy(), k)
