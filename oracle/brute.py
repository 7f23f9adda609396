"""Brute-force paged attention in pure Python.  TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Restates [Serving] The Build, Step 6 loop by loop, for tiny inputs only: walk the page
table block by block, within a block walk the stored tokens (the last block stops at the
sequence length), score each token against the query, softmax the scores, then walk the
pages again to add each value weighted by its softmax weight.  Per-head scores and the
GQA head mapping follow the readings in oracle/attention.py.

It shares nothing with oracle/attention.py: stored bits are widened with ``struct``,
products and sums use Python floats and ``math.exp``.  Its only role is to pin the
vectorised oracle on tiny shapes.
"""
from __future__ import annotations

import math
import struct


def _widen(bits: int, dtype: str) -> float:
    bits = int(bits)
    if dtype == "f32":
        return struct.unpack("<f", struct.pack("<I", bits))[0]
    if dtype == "bf16":
        return struct.unpack("<f", struct.pack("<I", bits << 16))[0]
    if dtype == "f16":
        return struct.unpack("<e", struct.pack("<H", bits))[0]
    raise ValueError(dtype)


def decode_one(q_bits_row, cache, table, L: int, h: int, num_q_heads: int, scale: float):
    """Output (list of floats) of query head ``h`` over the first ``L`` tokens of one sequence."""
    dt = cache.dtype
    bs = cache.bs
    G = num_q_heads // cache.H
    g = h // G
    D = cache.D
    q = [_widen(q_bits_row[d], dt) for d in range(D)]
    scores = [0.0] * L
    for logical, page in enumerate(table):
        start = logical * bs
        if start >= L:
            break
        end = min(start + bs, L)
        for t in range(start, end):
            off = t - start
            acc = 0.0
            for d in range(D):
                acc += q[d] * _widen(cache.k[page, g, off, d], dt)
            scores[t] = acc * scale
    top = max(scores)
    ex = [math.exp(s - top) for s in scores]
    z = sum(ex)
    w = [e / z for e in ex]
    out = [0.0] * D
    for logical, page in enumerate(table):
        start = logical * bs
        if start >= L:
            break
        end = min(start + bs, L)
        for t in range(start, end):
            off = t - start
            for d in range(D):
                out[d] += w[t] * _widen(cache.v[page, g, d, off], dt)
    return out, w
