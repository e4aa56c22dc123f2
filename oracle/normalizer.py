"""Log-sum-exp of each row of logits (oracle; test infrastructure only).

Selective Log Softmax page: a log-probability is the logit minus the row's
log-sum-exp over the whole vocabulary, log(sum_v exp(L[v])); its section
"Kernel design" reaches that value through per-slice maxima and sums, which
is only a way to evaluate the same definition.  Written out here in float64:
with M the largest logit, lse = M + log(sum_v exp(L[v] - M)) (exact up to
rounding; subtracting M keeps every exponential at most 1).  An +inf logit
makes lse +inf; a row of -inf logits has lse -inf (the sum is empty).

Parity status: pinned (closed forms log(V) and lse of one entry, shift
invariance, the brute-force log of a sum, an independent library routine;
tests/test_oracle_pins.py).
"""

import numpy as np


def logsumexp_row(row):
    """Log-sum-exp of one 1-D row of float logits, in float64."""
    x = np.asarray(row, dtype=np.float64)
    assert x.ndim == 1 and x.shape[0] >= 1
    top = x.max()
    if top == np.inf:
        return np.inf
    if top == -np.inf:
        return -np.inf
    return float(top + np.log(np.sum(np.exp(x - top))))


def logsumexp_rows(L):
    """logsumexp_row of every row of a 2-D array (float64 [M])."""
    L = np.asarray(L)
    return np.array([logsumexp_row(L[m]) for m in range(L.shape[0])], dtype=np.float64)
