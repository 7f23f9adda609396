"""Brute-force paged attention in pure Python.  TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

For tiny inputs only.  It is written from the definitions, with no vectorisation:

* where a token lives ([Serving] "Production Serving: Continuous Batching and PagedAttention",
  The Build, Step 4): logical position ``pos`` of a sequence is slot ``pos % block_size`` of the
  physical block ``table[pos // block_size]``;
* what attention computes (Step 6, with the per-head reading of oracle/attention.py):
  score_t = scale * sum_d q_d K_{t,d} for every stored position t < L of the query head's KV
  head, w_t = exp(score_t - max) / sum_u exp(score_u - max), out_d = sum_t w_t V_{t,d}.

It shares nothing with oracle/attention.py: stored bits are widened with ``struct``, products
and sums use Python floats, ``math.exp`` and the exactly rounded ``math.fsum``.  Its only role is
to pin the vectorised oracle on tiny shapes.
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


def _where(table, pos: int, block_size: int):
    """(physical block, slot) of logical position ``pos``."""
    return int(table[pos // block_size]), pos % block_size


def decode_one(q_bits_row, cache, table, L: int, h: int, num_q_heads: int, scale: float):
    """Output (list of floats) of query head ``h`` over the first ``L`` tokens of one sequence,
    and the softmax weights (list of floats, one per position)."""
    dt = cache.dtype
    D = cache.D
    g = h // (num_q_heads // cache.H)  # the query head's KV head
    q = [_widen(q_bits_row[d], dt) for d in range(D)]
    places = [_where(table, pos, cache.bs) for pos in range(L)]
    keys = [[_widen(cache.k[blk, g, off, d], dt) for d in range(D)] for blk, off in places]
    vals = [[_widen(cache.v[blk, g, d, off], dt) for d in range(D)] for blk, off in places]
    scores = [scale * math.fsum(q[d] * key[d] for d in range(D)) for key in keys]
    top = max(scores)
    num = [math.exp(s - top) for s in scores]
    den = math.fsum(num)
    w = [x / den for x in num]
    out = [math.fsum(w[t] * vals[t][d] for t in range(L)) for d in range(D)]
    return out, w
