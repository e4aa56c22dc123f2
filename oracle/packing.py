"""Binary-head packing (oracle; test infrastructure only).

pack_logical follows the lm-head-topk page, section "Usage" (signs with one
scale per group of 128 weights) and section "Requirements and limits"
(packing is an offline step before the fused call).  The pages fix neither
the sign of zero nor the scale rule; the readings used here are: the sign is
+1 exactly when the weight is >= 0 (so -0.0 gives +1), and the scale is the
mean absolute value of the group's 128 weights, summed in float64 and rounded
once to fp32.

pack_layout_bytes / unpack_layout_bytes write and read the library's packed
layout, version 1, from its specification (the "Packed binary head" comment of
include/lmtopk.h), in code of their own: plain index arithmetic, no shared
helpers with the HIP library.

Parity status: pinned (recovery of known signs and scales, hand-written golden
layout fixture; tests/test_oracle_pins.py).
"""

import numpy as np

GROUP = 128


def packed_sizes(V, H):
    """(wq_bytes, wscale_bytes) of a V x H head in layout version 1."""
    G = H // GROUP
    G4 = -(-G // 4) * 4
    V64 = -(-V // 64) * 64
    return V64 * H // 8, V64 * G4 * 4


def pack_logical(W):
    """Signs (int8, +1/-1) [V, H] and fp32 group scales [V, H/128] of a dense head.

    W: [V, H] fp32 (widen bf16 first).  Sign +1 iff W >= 0.  Scale of group g
    of row v: (sum over the group of |W| in float64) / 128, rounded to fp32.
    """
    W = np.asarray(W, dtype=np.float32)
    V, H = W.shape
    assert H % GROUP == 0
    signs = np.where(W >= 0, np.int8(1), np.int8(-1))
    # |w| is exact in fp32; each group is summed in float64
    sums = np.abs(W).reshape(V, H // GROUP, GROUP).sum(axis=2, dtype=np.float64)
    scales = (sums / GROUP).astype(np.float32)
    return signs, scales


def pack_layout_bytes(signs, scales):
    """Write logical (signs, scales) into layout version 1.

    Returns (wq as uint32 array, wscale as float32 array), both 1-D.  For row
    v = 64 t + r, group g, word w: the word at ((t*G + g)*64 + r)*4 + w has
    bit b set iff the sign of element 128 g + 32 w + b is +1.  The scale of
    group g = 4 q + i sits at ((t*(G4/4) + q)*64 + r)*4 + i.  Padding rows and
    groups stay 0.
    """
    signs = np.asarray(signs)
    scales = np.asarray(scales, dtype=np.float32)
    V, H = signs.shape
    G = H // GROUP
    G4 = -(-G // 4) * 4
    T = -(-V // 64)
    wq = np.zeros(T * G * 64 * 4, dtype=np.uint32)
    ws = np.zeros(T * (G4 // 4) * 64 * 4, dtype=np.float32)
    bitval = (np.uint64(1) << np.arange(32, dtype=np.uint64))
    for v in range(V):
        t, r = divmod(v, 64)
        pos = signs[v] > 0
        for g in range(G):
            for w in range(4):
                bits = pos[GROUP * g + 32 * w: GROUP * g + 32 * w + 32]
                word = int(np.sum(bitval[bits]))
                wq[((t * G + g) * 64 + r) * 4 + w] = word
            q, i = divmod(g, 4)
            ws[((t * (G4 // 4) + q) * 64 + r) * 4 + i] = scales[v, g]
    return wq, ws


def unpack_layout_bytes(wq, wscale, V, H):
    """Read layout version 1 back into logical (signs int8 [V,H], scales fp32 [V,G]).

    Vectorised reading of the same index rule as pack_layout_bytes.
    """
    G = H // GROUP
    G4 = -(-G // 4) * 4
    T = -(-V // 64)
    wq = np.asarray(wq).view(np.uint32).reshape(T, G, 64, 4)
    ws = np.asarray(wscale).view(np.float32).reshape(T, G4 // 4, 64, 4)
    # [T, G, 64, 4 words] -> [T, 64, G, 4 words] -> rows [T*64, G*4 words]
    words = wq.transpose(0, 2, 1, 3).reshape(T * 64, G * 4)[:V]
    shifts = np.arange(32, dtype=np.uint32)
    bits = (words[:, :, None] >> shifts[None, None, :]) & np.uint32(1)
    signs = np.where(bits.reshape(V, G * 4 * 32) == 1, 1, -1).astype(np.int8)
    sc = ws.transpose(0, 2, 1, 3).reshape(T * 64, G4)[:V, :G]
    return signs, np.ascontiguousarray(sc)
