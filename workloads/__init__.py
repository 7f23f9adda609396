"""Seeded synthetic inputs for paged decode attention, shared by tests, bench.py and smoke().

This module only draws inputs: context lengths, block free orders, K/V/Q values and
the request trace of a continuous-batching run.  It holds none of the method's
arithmetic (no pool logic, no slot arithmetic, no attention): the oracle and the HIP
path each implement that on their own and receive the same bytes from here.

Value recipe: fp32 draws from N(0, 1) with ``numpy.random.default_rng``, rounded to the
storage type on the host (bf16 by round-to-nearest-even on the fp32 bit pattern, fp16
by numpy's IEEE conversion).  Integer ranges are inclusive.  Raw storage bits are
returned (uint16 for bf16/fp16, uint32 for fp32) so that both sides see identical bytes.

Workload shapes follow the three pages on continuous batching and PagedAttention
(16-token blocks, block tables, per-step append then attend) and the five configs of
this library's benchmark list: tiny fp32 decode, a Llama-3-8B-shaped batch-64 decode,
a continuous-batching trace, a 32K long-context decode and a mixed prefix-sharing step.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

DTYPES = ("f32", "f16", "bf16")
BLOCK_SIZE = 16

# Quiet-NaN bit patterns used to pre-fill caches, so that a stray read of an unwritten
# slot poisons the result instead of passing silently.
NAN_BITS = {"bf16": 0x7FC0, "f16": 0x7E00, "f32": 0x7FC00000}


def storage_np_dtype(dtype: str):
    if dtype == "f32":
        return np.uint32
    if dtype in ("f16", "bf16"):
        return np.uint16
    raise ValueError(f"unknown dtype {dtype!r}")


def elem_bytes(dtype: str) -> int:
    return 4 if dtype == "f32" else 2


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even) and return the 16-bit patterns."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def f32_to_bits(x, dtype: str) -> np.ndarray:
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    if dtype == "f32":
        return x.view(np.uint32).copy()
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16).copy()
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(dtype)


def normal_bits(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0,1) fp32 draws rounded to ``dtype``; returns raw storage bits of ``shape``."""
    return f32_to_bits(rng.standard_normal(size=shape, dtype=np.float32), dtype)


def nan_filled(shape, dtype: str) -> np.ndarray:
    return np.full(shape, NAN_BITS[dtype], dtype=storage_np_dtype(dtype))


def blocks_for(n_tokens: int, block_size: int = BLOCK_SIZE) -> int:
    return -(-int(n_tokens) // block_size)


# --------------------------------------------------------------------------------------
# Decode-step workloads (tiny, Llama-shaped, long context)
# --------------------------------------------------------------------------------------
@dataclass
class DecodeWorkload:
    """One continuous-batching decode step: every sequence already holds ``lens - 1``
    cached tokens, appends one token, then attends over all ``lens`` tokens."""

    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    D: int
    dtype: str
    lens: np.ndarray  # int32 [B], context length after this step's append
    num_blocks: int
    free_order: np.ndarray  # int32 [num_blocks]; allocation pops from the end
    scale: float
    partition_size: int = 0  # 0: single pass
    block_size: int = BLOCK_SIZE
    extra: dict = field(default_factory=dict)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def max_blocks_per_seq(self) -> int:
        return blocks_for(int(self.lens.max()), self.block_size)

    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes one decode call reads: every cached token once per KV head."""
        return int(self.lens.astype(np.int64).sum()) * self.Hkv * self.D * 2 * elem_bytes(self.dtype)

    def q_bytes(self) -> int:
        return self.B * self.Hq * self.D * elem_bytes(self.dtype)


def tiny_decode(seed: int = 1) -> DecodeWorkload:
    """Tiny fp32 MHA step: batch 4, 8/8 heads of 64, pool of 32 blocks, lengths {5,17,32,40}."""
    rng = np.random.default_rng(seed)
    lens = np.array([5, 17, 32, 40], dtype=np.int32)
    free_order = rng.permutation(32).astype(np.int32)
    return DecodeWorkload("tiny_decode_b4_h8_d64_f32", seed, 4, 8, 8, 64, "f32", lens, 32,
                          free_order, 1.0 / math.sqrt(64), 0, extra={"rng": rng})


def llama_decode(seed: int = 2, B: int = 64, lo: int = 128, hi: int = 2048,
                 dtype: str = "bf16", partition_size: int = 512) -> DecodeWorkload:
    """Llama-3-8B-shaped decode layer: 32 q / 8 kv heads of 128, batch 64, L ~ U[128, 2048]
    inclusive; pool = total need + 10% (rounded up), handed out from a shuffled free list."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)
    need = int(sum(blocks_for(l) for l in lens))
    N = int(math.ceil(1.1 * need))
    free_order = rng.permutation(N).astype(np.int32)
    return DecodeWorkload(f"llama3_8b_decode_b{B}_gqa32x8_d128_{dtype}", seed, B, 32, 8, 128, dtype,
                          lens, N, free_order, 1.0 / math.sqrt(128), partition_size,
                          extra={"rng": rng})


def long_context_decode(seed: int = 4, B: int = 8, L: int = 32768,
                        partition_size: int = 512, dtype: str = "bf16") -> DecodeWorkload:
    """Long-context decode: batch 8 at 32,768 tokens, 2,048 scattered blocks each,
    split-K over 512-token partitions; pool = need + 10%."""
    rng = np.random.default_rng(seed)
    lens = np.full(B, L, dtype=np.int32)
    need = B * blocks_for(L)
    N = int(math.ceil(1.1 * need))
    free_order = rng.permutation(N).astype(np.int32)
    return DecodeWorkload(f"long_context_decode_b{B}_L{L}_gqa32x8_d128_{dtype}", seed, B, 32, 8, 128,
                          dtype, lens, N, free_order, 1.0 / math.sqrt(128), partition_size,
                          extra={"rng": rng})


def custom_decode(seed: int, lens, Hq: int, Hkv: int, D: int, dtype: str, num_blocks: int | None = None,
                  partition_size: int = 0, scale: float | None = None) -> DecodeWorkload:
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int32)
    need = int(sum(blocks_for(l) for l in lens))
    N = num_blocks if num_blocks is not None else int(math.ceil(1.1 * need)) + 1
    free_order = rng.permutation(N).astype(np.int32)
    return DecodeWorkload(f"custom_decode_s{seed}", seed, len(lens), Hq, Hkv, D, dtype, lens, N, free_order,
                          scale if scale is not None else 1.0 / math.sqrt(D), partition_size,
                          extra={"rng": rng})


@dataclass
class DecodeTensors:
    """Raw bits for one decode step, drawn in a fixed order after lengths and free order:
    cached-prefix K/V (per sequence, ``lens[b] - 1`` tokens), step K/V, then Q."""

    prefix_k: list  # per seq: [lens[b]-1, Hkv, D]
    prefix_v: list
    step_k: np.ndarray  # [B, Hkv, D]
    step_v: np.ndarray
    q: np.ndarray  # [B, Hq, D]


def decode_tensors(w: DecodeWorkload) -> DecodeTensors:
    rng = w.extra["rng"]
    pk, pv = [], []
    for b in range(w.B):
        n = int(w.lens[b]) - 1
        pk.append(normal_bits(rng, (n, w.Hkv, w.D), w.dtype))
        pv.append(normal_bits(rng, (n, w.Hkv, w.D), w.dtype))
    sk = normal_bits(rng, (w.B, w.Hkv, w.D), w.dtype)
    sv = normal_bits(rng, (w.B, w.Hkv, w.D), w.dtype)
    q = normal_bits(rng, (w.B, w.Hq, w.D), w.dtype)
    return DecodeTensors(pk, pv, sk, sv, q)


# --------------------------------------------------------------------------------------
# Continuous-batching trace
# --------------------------------------------------------------------------------------
@dataclass
class Request:
    rid: int
    arrival_step: int
    prompt_len: int
    output_len: int


def trace_requests(seed: int = 3, n: int = 512, prompt_median: int = 512, prompt_sigma: float = 1.0,
                   prompt_max: int = 8192, output_mean: int = 200, output_cap: int = 4096,
                   rate_per_step: float = 1.0) -> list:
    """Poisson arrivals (exponential gaps in scheduler steps, floored), lognormal prompt
    lengths clipped to [1, prompt_max], geometric output lengths (support >= 1) capped."""
    rng = np.random.default_rng(seed)
    gaps = rng.exponential(1.0 / rate_per_step, size=n)
    arrivals = np.floor(np.cumsum(gaps)).astype(np.int64)
    prompts = np.clip(np.round(rng.lognormal(math.log(prompt_median), prompt_sigma, size=n)),
                      1, prompt_max).astype(np.int64)
    outputs = np.minimum(rng.geometric(1.0 / output_mean, size=n), output_cap).astype(np.int64)
    return [Request(i, int(arrivals[i]), int(prompts[i]), int(outputs[i])) for i in range(n)]


def token_kv(seed: int, rid: int, start: int, count: int, Hkv: int, D: int, dtype: str):
    """K/V bits for tokens [start, start+count) of request ``rid``.  Each position has its own
    counter-keyed stream, so recomputing a preempted request reproduces the same bytes."""
    ks = np.empty((count, Hkv, D), dtype=storage_np_dtype(dtype))
    vs = np.empty_like(ks)
    for i in range(count):
        r = np.random.default_rng([seed, rid, start + i])
        ks[i] = normal_bits(r, (Hkv, D), dtype)
        vs[i] = normal_bits(r, (Hkv, D), dtype)
    return ks, vs


def token_kv_bulk(seed: int, rid: int, count: int, Hkv: int, D: int, dtype: str):
    """Prompt K/V bits of request ``rid`` (one stream for the whole prompt)."""
    r = np.random.default_rng([seed, rid, 1 << 40])
    return normal_bits(r, (count, Hkv, D), dtype), normal_bits(r, (count, Hkv, D), dtype)


def step_kv(seed: int, step: int, B: int, Hkv: int, D: int, dtype: str):
    """K/V bits of the B tokens a decode step appends (one stream per step)."""
    r = np.random.default_rng([seed, 1 << 42, step])
    return normal_bits(r, (B, Hkv, D), dtype), normal_bits(r, (B, Hkv, D), dtype)


def shuffled_free_order(seed: int, num_blocks: int) -> np.ndarray:
    """A seeded permutation of the pool's block ids (allocation pops from the end)."""
    return np.random.default_rng([seed, 1 << 43]).permutation(num_blocks).astype(np.int32)


def step_queries(seed: int, step: int, B: int, Hq: int, D: int, dtype: str):
    r = np.random.default_rng([seed, 1 << 41, step])
    return normal_bits(r, (B, Hq, D), dtype)


# --------------------------------------------------------------------------------------
# Mixed step with prefix sharing + chunked prefill
# --------------------------------------------------------------------------------------
@dataclass
class MixedWorkload:
    seed: int
    samples: int = 16
    prefix_len: int = 2048  # 2040 for the copy-on-write variant
    ctx_start: int = 4096
    chunk: int = 512
    token_budget: int = 2048
    Hq: int = 32
    Hkv: int = 8
    D: int = 128
    dtype: str = "bf16"
    num_blocks: int = 0
    free_order: np.ndarray = None
    scale: float = 1.0 / math.sqrt(128)


def mixed_step(seed: int = 5, prefix_len: int = 2048, samples: int = 16, ctx_start: int = 4096,
               chunk: int = 512) -> MixedWorkload:
    """16 samples share a refcounted prefix and each append one token; one prefill chunk of 512
    rows attends causally over a 4096-token paged context.  Pool = need + 10%."""
    w = MixedWorkload(seed, samples=samples, prefix_len=prefix_len, ctx_start=ctx_start, chunk=chunk)
    need = blocks_for(prefix_len) + samples + blocks_for(ctx_start + chunk)
    w.num_blocks = int(math.ceil(1.1 * need))
    rng = np.random.default_rng(seed)
    w.free_order = rng.permutation(w.num_blocks).astype(np.int32)
    w.rng = rng
    return w
