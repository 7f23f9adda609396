"""Oracle attention over the paged cache.  TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

What is computed, per [Serving] The Build, Step 6 (attention over paged storage): the
cached tokens of a sequence are found through its page table; every cached token gets a
score, the query dotted with the token's key divided by sqrt(head_dim); the scores go
through a softmax; the output is the weight-sum of the values.  Readings (the page's code
is garbled or silent here):

* Scores are per head: query head h is scored only against its own KV head (the page's
  sum runs over all heads at once, which would give one score per token for every head).
* Grouped-query attention ([Serving] Why It Matters names it as changing the cache shape):
  query head h uses KV head h // (num_q_heads / num_kv_heads).
* ``scale`` is passed in (1/sqrt(head_dim) in every workload).
* Only the ``L`` stored tokens take part: the unused tail of the last block is never read.
* A decode step attends over the context after that step's append (the new token attends
  to itself); for a prefill chunk, row i at absolute position ``ctx_start + i`` attends to
  positions 0 .. ctx_start + i (causal), per [Chapter] "How the scheduler works" and
  [Notes] "Prefill gets in the way" (a prompt is cut into chunks processed step by step).

Implementation: gather the blocks into contiguous K/V, decode the stored bits exactly to
fp64, then the textbook softmax(scale * K q) V with the maximum subtracted (exact in fp64).
The result does not depend on how a kernel partitions the context, so split-K has no
oracle of its own.
"""
from __future__ import annotations

import numpy as np


def bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored bits to fp64."""
    bits = np.asarray(bits)
    if dtype == "f32":
        return bits.astype(np.uint32).view(np.float32).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f16":
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    raise ValueError(dtype)


def gather(cache, table, L: int):
    """Contiguous fp64 K and V of one sequence: each [num_kv_heads][L][head_dim]."""
    bs = cache.bs
    nb = -(-int(L) // bs)
    blocks = np.asarray(table[:nb], dtype=np.int64)
    if nb and (blocks.min() < 0 or blocks.max() >= cache.N):
        raise IndexError("block table entry outside the pool")
    if cache.dtype == "fp8":  # codes times their per-slot scales, exact in fp64
        k, v = cache.dequant_kv(blocks)
    else:
        k = bits_to_f64(cache.k[blocks], cache.dtype)  # [nb][H][bs][D]
        v = bits_to_f64(cache.v[blocks], cache.dtype)  # [nb][H][D][bs]
    K = k.transpose(1, 0, 2, 3).reshape(cache.H, nb * bs, cache.D)[:, :L]
    V = v.transpose(1, 0, 3, 2).reshape(cache.H, nb * bs, cache.D)[:, :L]
    return K, V


def softmax_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """One query row against L keys/values: returns (output [D], weights [L])."""
    s = scale * (K @ q)
    s = s - s.max()
    e = np.exp(s)
    w = e / e.sum()
    return w @ V, w


def paged_decode(q_bits, cache, tables, lens, scale: float, return_weights: bool = False, q_dtype=None):
    """Decode attention for a batch.  q_bits [B][Hq][D] (of q_dtype, default the cache's type);
    tables rows of physical block ids; lens[b] >= 1 tokens.  Returns fp64 [B][Hq][D] (and per-(b, h)
    weights on request)."""
    q = bits_to_f64(q_bits, q_dtype or cache.dtype)
    B, Hq, D = q.shape
    if Hq % cache.H:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // cache.H
    out = np.zeros((B, Hq, D), dtype=np.float64)
    weights = {}
    for b in range(B):
        L = int(lens[b])
        if L < 1:
            raise ValueError("context length must be >= 1")
        K, V = gather(cache, tables[b], L)
        for h in range(Hq):
            g = h // G
            out[b, h], w = softmax_attention(q[b, h], K[g], V[g], scale)
            if return_weights:
                weights[(b, h)] = w
    return (out, weights) if return_weights else out


def prefill_chunk(q_bits, cache, table, ctx_start: int, scale: float, q_dtype=None):
    """Causal attention of a prompt chunk against the paged cache: q_bits [C][Hq][D] (of q_dtype,
    default the cache's type; an fp8 cache needs bf16 or f16 queries), row i sits at position
    ctx_start + i and sees keys 0 .. ctx_start + i.  Returns fp64 [C][Hq][D]."""
    q = bits_to_f64(q_bits, q_dtype or cache.dtype)
    C, Hq, D = q.shape
    G = Hq // cache.H
    K, V = gather(cache, table, ctx_start + C)
    out = np.zeros((C, Hq, D), dtype=np.float64)
    for i in range(C):
        n = ctx_start + i + 1
        for h in range(Hq):
            g = h // G
            out[i, h], _ = softmax_attention(q[i, h], K[g, :n], V[g, :n], scale)
    return out
