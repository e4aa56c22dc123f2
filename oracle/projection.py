"""Vocabulary projection in float64 (oracle; test infrastructure only).

Parity status: pinned.  Closed forms, exact integer arithmetic and a worked
example pin every function here (tests/test_oracle_pins.py).
"""

import numpy as np

GROUP = 128


def bf16_bits_to_f32(bits):
    """Widen bf16 values (given as their uint16 bit patterns) to fp32.

    A bf16 number is the upper half of an IEEE fp32 number, so placing its 16
    bits in the high half of a 32-bit word gives the same value exactly.
    """
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def project_dense(hidden, weight, bias=None, block_rows=4096):
    """Dense head logits L[m, v] = sum_j hidden[m, j] * weight[v, j] + bias[v].

    lm-head-topk page, section "Usage": the dense entry point takes the
    hidden rows and the head's weight matrix [V, H]; section "Correctness":
    with and without bias.  Inputs are fp32 arrays (widen bf16 first with
    bf16_bits_to_f32); the sum is taken in float64 over blocks of vocabulary
    rows.  Returns float64 [M, V].
    """
    h = np.asarray(hidden, dtype=np.float64)
    w = np.asarray(weight)
    M, H = h.shape
    V, H2 = w.shape
    assert H == H2, "hidden and weight disagree on H"
    out = np.empty((M, V), dtype=np.float64)
    for v0 in range(0, V, block_rows):
        blk = w[v0:v0 + block_rows].astype(np.float64)
        out[:, v0:v0 + blk.shape[0]] = h @ blk.T
    if bias is not None:
        out += np.asarray(bias, dtype=np.float64)[None, :]
    return out


def project_binary(act_q, act_scale, signs, scales, bias=None, block_rows=4096):
    """Binary head logits, the "dequantized reference" of the lm-head-topk page.

    lm-head-topk page, section "Usage" (act_q, act_scale, packed signs with
    per-group scales, optional bias) and section "Correctness" (binary values
    are checked against a dequantized reference):
        L[m, v] = sum_j (act_q[m, j] * act_scale[m]) * (sign[v, j] * scale[v, j // 128])
                  + bias[v]
    computed in float64 over blocks of vocabulary rows.  Returns [M, V].
    """
    a = np.asarray(act_q).astype(np.float64)
    x = a * np.asarray(act_scale, dtype=np.float64)[:, None]
    s = np.asarray(signs)
    sc = np.asarray(scales, dtype=np.float32)
    V, H = s.shape
    assert x.shape[1] == H and H % GROUP == 0
    out = np.empty((x.shape[0], V), dtype=np.float64)
    buf = np.empty((min(block_rows, V), H), dtype=np.float64)
    for v0 in range(0, V, block_rows):
        n = min(block_rows, V - v0)
        wd = buf[:n]
        # dequantized block, written in place: sign[v, j] * scale[v, j // 128]
        np.multiply(s[v0:v0 + n].reshape(n, H // GROUP, GROUP),
                    sc[v0:v0 + n, :, None].astype(np.float64),
                    out=wd.reshape(n, H // GROUP, GROUP))
        out[:, v0:v0 + n] = x @ wd.T
    if bias is not None:
        out += np.asarray(bias, dtype=np.float64)[None, :]
    return out
