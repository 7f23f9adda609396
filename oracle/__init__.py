"""CPU oracle for paged KV-cache decode attention.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package.  The product (``paged_kv_cache_404_amd``) never imports it, and this
package imports nothing from the product: the two share no code.  The only common module
is ``workloads`` (seeded input generators, no method arithmetic).

It is a plain, slow, obviously correct restatement of what the method computes, written in
Python + numpy, floating point in fp64.  Sources, cited by page title and section:

* [Serving] "Production Serving: Continuous Batching and PagedAttention"
  (llm-under-the-hood, project 17): The Concept; The Build, Step 4 (paged KV cache:
  block pool, page table, append, free), Step 6 (attention over paged storage),
  Step 8 (prefix caching).
* [Chapter] "Continuous batching and PagedAttention" (how-ai-works, chapter 7):
  "How the scheduler works" (chunked prefill), "PagedAttention: KV cache memory"
  (16-token blocks, copy-on-write sharing, preemption).
* [Notes] "Continuous batching and PagedAttention: serving many users from one GPU"
  (trefon notes): "Fragmentation: PagedAttention" (block table, sharing until
  divergence), "Prefill gets in the way" (chunked prefill), "Memory, not compute, caps
  the batch" (quantised caches hold more tokens).
* The FP8 format itself is the OCP 8-bit Floating Point Specification's E4M3 (not on the pages).

Modules:
  pool       host block pool model: LIFO free list, refcounts, fork, copy-on-write,
             all-or-nothing append, free, block tables and slot mapping
  cache      byte-exact model of the paged K/V cache layout, append and block copy
  attention  gather to contiguous K/V and fp64 softmax attention (decode, prefill chunk)
  fp8        FP8 (OCP E4M3) K/V cache: codec, per-(token, head) quantisation, cache model
  brute      pure-Python per-page / per-token loops for tiny inputs (pins the numpy path)

Pins: every function here is checked in ``tests/test_oracle_*.py`` against values the pages
fix, closed forms, invariants and brute force.  None of the pages prints an attention value
or a worked attention example, so attention is pinned by the other kinds: closed forms
(one-token context = V, constant V, zero query = mean of V), invariants (physical-block
permutation, softmax weights summing to 1, GQA = MHA on repeated K/V), brute force on tiny
inputs, and torch's scaled-dot-product attention as an independent library routine.
"""

from .pool import PoolModel, OutOfBlocks, InvalidOp  # noqa: F401
from .cache import CacheModel  # noqa: F401
from .fp8 import Fp8CacheModel  # noqa: F401
from . import attention, brute, fp8  # noqa: F401
