"""Grammar bitmask applied to logits (oracle; test infrastructure only).

logits-processor page, section "API": a bitmask of int32 words [B,
ceil(V/32)] marks the allowed tokens with bit 1 (the XGrammar convention)
and every disallowed logit is set to -inf.  Bit (v mod 32) of word v div 32
belongs to vocabulary entry v (bits past V unused).  Applying the mask and
then taking the top-k or the log-sum-exp of the result is the definition the
library's masked calls must reach.

Parity status: pinned (hand-worked words, the all-ones and all-zero masks, a
mask built by NumPy's independent bit packing; tests/test_oracle_pins.py).
"""

import numpy as np


def allowed_bool(bitmask, V):
    """[M, ceil(V/32)] int32 words -> [M, V] bool, entry v allowed iff its bit is 1."""
    words = np.asarray(bitmask).astype(np.int64) & 0xFFFFFFFF
    M = words.shape[0]
    out = np.zeros((M, V), dtype=bool)
    for v in range(V):
        out[:, v] = (words[:, v // 32] >> (v % 32)) & 1 == 1
    return out


def apply_allowed(L, bitmask):
    """Copy of logits L [M, V] with every disallowed entry set to -inf."""
    L = np.array(L, copy=True)
    L[~allowed_bool(bitmask, L.shape[1])] = -np.inf
    return L
