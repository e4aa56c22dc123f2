"""Exact top-k selection (oracle; test infrastructure only).

lm-head-topk page, section "API": the result is (values, indices) sorted by
value descending; section "Method", last sentence: equal values resolve to the
lower vocabulary index.  That is the total order (value desc, index asc), and
a stable sort of the negated values realises it.  +0.0 and -0.0 compare equal
here (NumPy's sort compares with <), so they tie and the lower index wins.

Parity status: pinned (brute-force ranking, argmax, hand-worked golden case;
tests/test_oracle_pins.py).
"""

import numpy as np


def topk_stable(row, k):
    """Indices (int64) and values of the k largest entries of one row.

    row: 1-D float array (any float dtype; compared in its own precision,
    which is exact for fp32 and fp64 alike).  The values returned are row's
    own entries at those indices, bit for bit.
    """
    row = np.asarray(row)
    assert row.ndim == 1 and 1 <= k <= row.shape[0]
    order = np.argsort(-row, kind="stable")[:k].astype(np.int64)
    return row[order], order


def topk_stable_rows(L, k):
    """topk_stable applied to every row of a 2-D array; returns (values, indices)."""
    L = np.asarray(L)
    vals = np.empty((L.shape[0], k), dtype=L.dtype)
    idx = np.empty((L.shape[0], k), dtype=np.int64)
    for m in range(L.shape[0]):
        vals[m], idx[m] = topk_stable(L[m], k)
    return vals, idx


def float_key_order(a, b, ia, ib):
    """True if (a, ia) comes before (b, ib) in the output order.

    Larger value first; equal values (with +0.0 == -0.0) put the lower index
    first.
    """
    if a != b:
        return a > b
    return ia < ib


def certify_topk(row, values, indices, k):
    """Sort-free check that (values, indices) is the exact top-k of row.

    The four conditions together define the result uniquely:
      1. k distinct indices, all in [0, V);
      2. values[i] is bitwise row[indices[i]];
      3. the pairs are in output order (value desc, index asc);
      4. every index j left out comes after the last pair: row[j] < v_k, or
         row[j] == v_k and j > i_k.
    Returns (ok, reason).
    """
    row = np.asarray(row)
    values = np.asarray(values)
    indices = np.asarray(indices).astype(np.int64)
    V = row.shape[0]
    if values.shape != (k,) or indices.shape != (k,):
        return False, "shape"
    if np.any(indices < 0) or np.any(indices >= V):
        return False, "index out of range"
    if np.unique(indices).shape[0] != k:
        return False, "duplicate index"
    got = row[indices]
    if not np.array_equal(got.view(np.uint8), values.astype(row.dtype).view(np.uint8)):
        return False, "value is not the row's entry"
    for i in range(k - 1):
        if not float_key_order(got[i], got[i + 1], indices[i], indices[i + 1]):
            return False, f"not in output order at {i}"
    vk, ik = got[-1], indices[-1]
    rest = np.ones(V, dtype=bool)
    rest[indices] = False
    j = np.nonzero(rest)[0]
    rj = row[j]
    bad = (rj > vk) | ((rj == vk) & (j < ik))
    if np.any(bad):
        return False, f"left-out index {int(j[np.argmax(bad)])} beats the k-th"
    return True, ""
