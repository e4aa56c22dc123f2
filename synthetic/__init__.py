"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module draws random numbers and prepares inputs; it holds none of the
method's arithmetic (no projection, no selection, no packing).  Both the CPU
oracle and the HIP library consume exactly the arrays produced here.

Recipe (the pages' workloads have no public dataset; these stand in for a
trained head at the pages' shapes):
  * every stream is numpy's PCG64 seeded with SeedSequence([seed, stream, block]),
    so blocks of rows can be drawn in parallel threads and the result does not
    depend on the thread count;
  * hidden rows and dense head rows are i.i.d. N(0,1) scaled by 1/sqrt(H),
    drawn in fp32 (the scale is rounded to fp32 once, the product once);
  * int8 activations are the hidden rows quantized symmetrically per row:
    scale = max|x| / 127 (fp32), q = round-half-even(x / scale) clipped to
    [-127, 127]; an all-zero row gets scale 1 and q = 0;
  * bias is i.i.d. N(0, 0.1^2) in fp32;
  * bf16 inputs are fp32 rounded to nearest-even and kept as uint16 bits.
"""

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

STREAM_HIDDEN = 0
STREAM_WEIGHT = 1
STREAM_BIAS = 2
STREAM_EXTRA = 3

BLOCK_ROWS = 8192


def _rng(seed, stream, block):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, block])))


def _threads():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_rows(rows, cols, seed, stream, scale=1.0, out=None, threads=None):
    """[rows, cols] fp32 of N(0,1) * fp32(scale), drawn in blocks of BLOCK_ROWS rows."""
    if out is None:
        out = np.empty((rows, cols), dtype=np.float32)
    assert out.shape == (rows, cols) and out.dtype == np.float32
    s = np.float32(scale)
    nblk = -(-rows // BLOCK_ROWS)

    def fill(b):
        sl = out[b * BLOCK_ROWS:(b + 1) * BLOCK_ROWS]
        _rng(seed, stream, b).standard_normal(out=sl, dtype=np.float32)
        if s != np.float32(1.0):
            np.multiply(sl, s, out=sl)

    n = threads or _threads()
    if nblk <= 1 or n == 1:
        for b in range(nblk):
            fill(b)
    else:
        with ThreadPoolExecutor(max_workers=n) as ex:
            list(ex.map(fill, range(nblk)))
    return out


def hidden_rows(M, H, seed=0):
    """Decode-row hidden vectors: N(0,1)/sqrt(H), fp32 [M, H]."""
    return normal_rows(M, H, seed, STREAM_HIDDEN, 1.0 / math.sqrt(H))


def dense_head(V, H, seed=0, out=None):
    """Head weights before any packing: N(0,1)/sqrt(H), fp32 [V, H]."""
    return normal_rows(V, H, seed, STREAM_WEIGHT, 1.0 / math.sqrt(H), out=out)


def bias_vector(V, seed=0, std=0.1):
    """Bias N(0, std^2), fp32 [V]."""
    return normal_rows(1, V, seed, STREAM_BIAS, std)[0].copy()


def quantize_rows_int8(x):
    """Symmetric per-row int8 quantization of fp32 rows: (q int8 [M,H], scale fp32 [M])."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=1)
    scale = (amax / np.float32(127.0)).astype(np.float32)
    zero = amax == 0
    scale[zero] = np.float32(1.0)
    q = np.rint(x / scale[:, None]).astype(np.float32)
    q = np.clip(q, -127, 127).astype(np.int8)
    q[zero] = 0
    return q, scale


def f32_to_bf16_bits(x):
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return rounded.astype(np.uint16)


def planted_bias(V, rows, value=5.0):
    """fp32 bias that is `value` on the given rows and 0 elsewhere."""
    b = np.zeros(V, dtype=np.float32)
    b[np.asarray(rows)] = np.float32(value)
    return b


def random_logits(M, V, seed=0, ties=0, signed_zeros=False):
    """fp32 logits [M, V] for the selection-only path.

    N(0,1) draws; with ties > 0 every value is rounded to a grid of `ties`
    distinct levels so exact ties are frequent; signed_zeros scatters +0.0 and
    -0.0 over ~1/8 of the entries each.
    """
    x = normal_rows(M, V, seed, STREAM_EXTRA)
    if ties:
        x = np.floor(x * np.float32(ties / 6.0)).astype(np.float32)
    if signed_zeros:
        r = _rng(seed, STREAM_EXTRA, 1 << 20).integers(0, 8, size=x.shape)
        x[r == 0] = np.float32(0.0)
        x[r == 1] = np.float32(-0.0)
    return x
