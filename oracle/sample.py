"""Sampling one token from the top-k survivors (oracle; test infrastructure only).

What is computed (logits-processor page, sections "API" and "Method"): one
logits -> token step made of temperature scaling, the intersection of the
top-k, top-p and min-p filters, and a draw.  top_k <= 0, top_p >= 1 and
min_p <= 0 each switch their filter off; temperature <= 0 means greedy.  Each
parameter may differ per row.  The draw is counter-based and keyed by
(seed, row, offset), so it is deterministic and can be replayed; the token is
drawn by the Gumbel-max trick over the kept set: argmax of (scaled logit +
Gumbel noise) picks token i with probability exp(z_i) / sum over the kept
set of exp(z_j).

Here the draw is fused after the exact top-k, so it sees the k survivors of
the call (sorted by value descending, lower index first on ties), and top-p
uses the normalizer over the WHOLE vocabulary.  Readings of the pages taken
here (they leave these steps open):

  * z = L / T are the scaled logits; lse_T = log sum_v exp(L[v] / T) over all
    V entries of the row (disallowed entries of a bitmask are -inf and add
    nothing); the probability of survivor i is p_i = exp(z_i - lse_T).
  * The keep set is a prefix of the survivors in output order: position 0 is
    always kept; position i >= 1 is kept while every earlier position was and
      - i < top_k (top_k <= 0 or top_k > k: i < k, the call's k),
      - the probability of the positions before it, p_0 + ... + p_{i-1}, is
        below top_p (when top_p < 1),
      - p_i / p_0 = exp(z_i - z_0) is at least min_p (when min_p > 0),
      - z_i is not -inf.
    Each filter keeps the most probable tokens above a cutoff, so they meet
    in one prefix (section "Method"); ties in probability are cut in the
    library's output order (lower vocabulary index first).
  * temperature <= 0: greedy, the token is the first survivor (the argmax,
    lower index on ties) and the keep set has size 1.  The same holds when
    the largest logit is +inf or every logit is -inf (no finite
    distribution exists).
  * The random numbers: Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
    "Parallel random numbers: as easy as 1, 2, 3", SC 2011) with key
    (seed mod 2^32, seed div 2^32) and counter (v, row, offset mod 2^32,
    offset div 2^32) for vocabulary entry v; its first output word x gives
    u = (floor(x / 2^9) + 1/2) * 2^-23, a uniform in (0, 1) that fp32 and
    fp64 both hold exactly; the noise is g = -log(-log(u)).
  * The token is the survivor with the largest z_i + g_i among the kept
    positions (the lower position on an exact tie).

Everything is float64.  Parity status: pinned (Philox known-answer vectors,
closed forms of the uniform and the noise, hand-worked keep sets, the
single-cutoff formulation of the filters, the Gumbel-max distribution by a
chi-square test; tests/test_oracle_pins.py).
"""

import math

import numpy as np

from .normalizer import logsumexp_row
from .select import topk_stable

MASK32 = 0xFFFFFFFF
# Philox4x32 round multipliers and key increments (the published constants:
# the multipliers of the paper, the increments are the golden ratio and
# sqrt(3) - 1 in 32-bit fixed point)
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85


def philox4x32_10(counter, key):
    """Philox4x32 with 10 rounds: four 32-bit counter words and two 32-bit
    key words -> four 32-bit output words (Python ints).

    One round: multiply counter words 0 and 2 by the two multipliers into
    64-bit products (hi, lo); the new words are (hi of product 2 ^ word 1 ^
    key 0, lo of product 2, hi of product 0 ^ word 3 ^ key 1, lo of product
    0).  The key advances by the two increments before every round after the
    first.
    """
    c0, c1, c2, c3 = (int(c) & MASK32 for c in counter)
    k0, k1 = (int(k) & MASK32 for k in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + PHILOX_W0) & MASK32
            k1 = (k1 + PHILOX_W1) & MASK32
        p0 = PHILOX_M0 * c0
        p1 = PHILOX_M1 * c2
        c0, c1, c2, c3 = ((p1 >> 32) ^ c1 ^ k0, p1 & MASK32, (p0 >> 32) ^ c3 ^ k1, p0 & MASK32)
    return c0, c1, c2, c3


def uniform_from_word(x):
    """A 32-bit word -> u in (0, 1): its top 23 bits plus one half, times 2^-23."""
    return (float((int(x) & MASK32) >> 9) + 0.5) * 2.0 ** -23


def draw_uniform(seed, row, offset, v):
    """The uniform the draw uses for vocabulary entry v of `row`."""
    seed, offset = int(seed), int(offset)
    x = philox4x32_10((v, row, offset & MASK32, offset >> 32), (seed & MASK32, seed >> 32))[0]
    return uniform_from_word(x)


def gumbel(u):
    """Standard Gumbel noise from a uniform in (0, 1)."""
    return -math.log(-math.log(u))


def keep_count(z, lse, top_k, top_p, min_p):
    """Size of the kept prefix of survivors with scaled logits z (output order).

    z: float64 [k], non-increasing; lse: log-normalizer of the scaled logits
    over the whole vocabulary.  Returns n in [1, k].
    """
    k = len(z)
    limit = k if top_k <= 0 else min(int(top_k), k)
    if not math.isfinite(z[0]):
        return 1
    n = 1
    below = math.exp(z[0] - lse)  # probability of the positions before n
    while n < limit:
        zi = z[n]
        if zi == -math.inf:
            break
        if top_p < 1.0 and below >= top_p:
            break
        if min_p > 0.0 and math.exp(zi - z[0]) < min_p:
            break
        below += math.exp(zi - lse)
        n += 1
    return n


def sample_row(L_row, k, temperature, top_k, top_p, min_p, seed, row, offset):
    """The draw for one row of logits L_row [V] (bitmask already applied).

    Returns a dict: token, kept (keep-set size), indices and values of the k
    survivors, z (their scaled logits), lse (normalizer of the scaled logits,
    None when greedy) and score (z + Gumbel noise of the kept positions).
    """
    L_row = np.asarray(L_row, dtype=np.float64)
    values, indices = topk_stable(L_row, k)
    out = {"indices": indices, "values": values}
    T = float(temperature)
    if T <= 0.0 or not math.isfinite(values[0]):
        out.update(token=int(indices[0]), kept=1, z=None, lse=None, score=None)
        return out
    z = values / T
    lse = logsumexp_row(L_row / T)
    n = keep_count(z, lse, top_k, top_p, min_p)
    score = np.array([z[i] + gumbel(draw_uniform(seed, row, offset, int(indices[i])))
                      for i in range(n)])
    best = int(np.argmax(score))  # first maximum: the lower position
    out.update(token=int(indices[best]), kept=n, z=z, lse=lse, score=score)
    return out


def _per_row(x, M, dtype):
    a = np.asarray(x, dtype=dtype)
    return np.broadcast_to(a, (M,)) if a.ndim == 0 else a


def sample_rows(L, k, temperature=1.0, top_k=0, top_p=1.0, min_p=0.0, seed=0, offset=0):
    """sample_row for every row of L [M, V]; each parameter a scalar or [M].

    Returns (tokens int64 [M], kept int64 [M]).
    """
    L = np.asarray(L, dtype=np.float64)
    M = L.shape[0]
    T = _per_row(temperature, M, np.float64)
    tk = _per_row(top_k, M, np.int64)
    tp = _per_row(top_p, M, np.float64)
    mp = _per_row(min_p, M, np.float64)
    tokens = np.empty(M, dtype=np.int64)
    kept = np.empty(M, dtype=np.int64)
    for m in range(M):
        r = sample_row(L[m], k, T[m], tk[m], tp[m], mp[m], seed, m, offset)
        tokens[m], kept[m] = r["token"], r["kept"]
    return tokens, kept
