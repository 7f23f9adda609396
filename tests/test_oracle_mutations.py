"""Planted mistakes in the oracle (CPU only): each plausible slip must fail at least one pin.

Every case swaps one oracle function for a copy carrying a single mistake, runs the pins
that should catch it, and asserts that at least one of them fails.  Nothing here touches
the HIP path.
"""
import numpy as np
import pytest

import oracle.attention as att
import oracle.cache as ocache
import oracle.fp8 as ofp8
import oracle.pool as opool
import tests.test_oracle_attention as TA
import tests.test_oracle_fp8 as TF
import tests.test_oracle_pool as TP


def _fails(*pins):
    failed = 0
    for pin in pins:
        try:
            pin()
        except (AssertionError, IndexError, ValueError, opool.OutOfBlocks, opool.InvalidOp):
            failed += 1
    return failed


def _softmax_no_scale(q, K, V, scale):
    s = K @ q
    s = s - s.max()
    e = np.exp(s)
    w = e / e.sum()
    return w @ V, w


def _softmax_sign_flip(q, K, V, scale):
    s = -scale * (K @ q)
    s = s - s.max()
    e = np.exp(s)
    w = e / e.sum()
    return w @ V, w


def _gather_v_untransposed(cache, table, L):
    bs = cache.bs
    nb = -(-int(L) // bs)
    blocks = np.asarray(table[:nb], dtype=np.int64)
    k = cache.k[blocks]
    v = cache.v[blocks]
    K = k.transpose(1, 0, 2, 3).reshape(cache.H, nb * bs, cache.D)[:, :L]
    V = v.transpose(1, 0, 2, 3).reshape(cache.H, nb * bs, cache.D)[:, :L]  # wrong axis order
    return att.bits_to_f64(K, cache.dtype), att.bits_to_f64(V, cache.dtype)


def _decode_gqa_modulo(q_bits, cache, tables, lens, scale, return_weights=False):
    q = att.bits_to_f64(q_bits, cache.dtype)
    B, Hq, D = q.shape
    out = np.zeros((B, Hq, D))
    for b in range(B):
        K, V = att.gather(cache, tables[b], int(lens[b]))
        for h in range(Hq):
            g = h % cache.H  # wrong head mapping
            out[b, h], _ = att.softmax_attention(q[b, h], K[g], V[g], scale)
    return out


def _prefill_off_by_one(q_bits, cache, table, ctx_start, scale):
    q = att.bits_to_f64(q_bits, cache.dtype)
    C, Hq, D = q.shape
    G = Hq // cache.H
    K, V = att.gather(cache, table, ctx_start + C)
    out = np.zeros((C, Hq, D))
    for i in range(C):
        n = max(1, ctx_start + i)  # drops the diagonal
        for h in range(Hq):
            out[i, h], _ = att.softmax_attention(q[i, h], K[h // G, :n], V[h // G, :n], scale)
    return out


@pytest.mark.parametrize("mutant", [_softmax_no_scale, _softmax_sign_flip])
def test_softmax_mutants_caught(monkeypatch, mutant):
    monkeypatch.setattr(att, "softmax_attention", mutant)
    assert _fails(TA.test_matches_torch_sdpa_fp64, TA.test_two_token_closed_form,
                  TA.test_huge_scale_selects_argmax_token) >= 1


def test_untransposed_v_caught(monkeypatch):
    monkeypatch.setattr(att, "gather", _gather_v_untransposed)
    assert _fails(TA.test_gather_round_trip_recovers_tokens_in_order,
                  lambda: TA.test_numpy_oracle_equals_brute_force("bf16", 4, 2, 8)) >= 1


def test_tail_read_caught(monkeypatch):
    orig = att.gather

    def reads_tail(cache, table, L):
        nb = -(-int(L) // cache.bs)
        return orig(cache, list(table) + [], nb * cache.bs)

    monkeypatch.setattr(att, "gather", reads_tail)
    assert _fails(TA.test_stale_tail_slots_are_never_read, TA.test_matches_torch_sdpa_fp64) >= 1


def test_gqa_mapping_mutant_caught(monkeypatch):
    monkeypatch.setattr(att, "paged_decode", _decode_gqa_modulo)
    assert _fails(TA.test_gqa_equals_mha_on_repeated_kv,
                  lambda: TA.test_numpy_oracle_equals_brute_force("bf16", 8, 2, 4)) >= 1


def test_causal_off_by_one_caught(monkeypatch):
    monkeypatch.setattr(att, "prefill_chunk", _prefill_off_by_one)
    assert _fails(TA.test_prefill_rows_equal_decodes_and_sdpa_causal,
                  TA.test_prefill_first_row_of_empty_context_returns_v) >= 1


def test_fifo_free_list_caught(monkeypatch):
    def fifo_alloc(self):
        if not self.free:
            raise opool.OutOfBlocks()
        b = self.free.pop(0)
        self.refcnt[b] = 1
        return b

    monkeypatch.setattr(opool.PoolModel, "_alloc", fifo_alloc)
    assert _fails(TP.test_alloc_pops_from_end_of_free_list, TP.test_tiny_step_worked_tables,
                  TP.test_free_returns_blocks_in_table_order) >= 1


def test_missing_copy_on_write_caught(monkeypatch):
    def blocks_needed_no_cow(self, seq, n):
        start = self.lens[seq]
        return sum(1 for pos in range(start, start + n) if pos % self.block_size == 0)

    def append_in_place(self, seq, n):
        need = blocks_needed_no_cow(self, seq, n)
        if need > len(self.free):
            raise opool.OutOfBlocks()
        table = self.tables[seq]
        slots = []
        for _ in range(n):
            pos = self.lens[seq]
            if pos % self.block_size == 0:
                table.append(self._alloc())
            slots.append(table[pos // self.block_size] * self.block_size + pos % self.block_size)
            self.lens[seq] = pos + 1
        return slots, []

    monkeypatch.setattr(opool.PoolModel, "append", append_in_place)
    monkeypatch.setattr(opool.PoolModel, "blocks_needed", blocks_needed_no_cow)
    assert _fails(TP.test_fork_shares_and_cow_isolates, TP.test_sixteen_samples_on_partial_prefix) >= 1


def test_free_order_reversed_caught(monkeypatch):
    def free_reversed(self, seq):
        idle = []
        for b in reversed(self.tables[seq]):
            self._release(b, idle)
        self.lru.extend(reversed(idle))
        del self.tables[seq]
        del self.lens[seq]

    monkeypatch.setattr(opool.PoolModel, "free_seq", free_reversed)
    assert _fails(TP.test_free_returns_blocks_in_table_order) >= 1


# ---- prefix cache ---------------------------------------------------------------------------
PREFIX_PINS = (TP.test_prefix_cache_worked_scenario, TP.test_prefix_cache_shares_the_common_first_block,
               TP.test_prefix_cache_capacity_counts_the_lru, TP.test_prefix_cache_random_invariants,
               TP.test_prefix_cache_eviction_unregisters_the_blocks_below)


def test_prefix_lookup_shortest_first_caught(monkeypatch):
    def lookup_shortest(self, tokens):
        s = self.new_seq()
        bs = self.block_size
        for n in range(bs, len(tokens) // bs * bs + 1, bs):
            key = tuple(int(t) for t in tokens[:n])
            if key in self.entries:
                for b in self.entries[key]:
                    if self.refcnt[b] == 0:
                        self.lru.remove(b)
                    self.refcnt[b] += 1
                self.tables[s] = list(self.entries[key])
                self.lens[s] = n
                return s, n
        return s, 0

    monkeypatch.setattr(opool.PoolModel, "prefix_lookup", lookup_shortest)
    assert _fails(*PREFIX_PINS) >= 1


def test_prefix_release_in_table_order_caught(monkeypatch):
    def free_table_order(self, seq):
        idle = []
        for b in self.tables[seq]:
            self._release(b, idle)
        self.lru.extend(idle)
        del self.tables[seq]
        del self.lens[seq]

    monkeypatch.setattr(opool.PoolModel, "free_seq", free_table_order)
    assert _fails(*PREFIX_PINS) >= 1


def test_prefix_eviction_keeps_descendants_caught(monkeypatch):
    def evict_only_exact(self):
        b = self.lru.pop(0)
        for key in [k for k, blocks in self.entries.items() if blocks[-1] == b]:
            del self.entries[key]
        return b

    monkeypatch.setattr(opool.PoolModel, "_evict", evict_only_exact)
    assert _fails(*PREFIX_PINS) >= 1


def test_prefix_hit_without_reference_caught(monkeypatch):
    orig = opool.PoolModel.prefix_lookup

    def lookup_no_ref(self, tokens):
        before = list(self.refcnt)
        lru = list(self.lru)
        s, n = orig(self, tokens)
        self.refcnt = before
        self.lru = lru
        return s, n

    monkeypatch.setattr(opool.PoolModel, "prefix_lookup", lookup_no_ref)
    assert _fails(*PREFIX_PINS) >= 1


def test_prefix_lru_freed_to_free_list_caught(monkeypatch):
    def release_always_free(self, b, idle):
        self.refcnt[b] -= 1
        if self.refcnt[b] == 0:
            self.free.append(b)

    monkeypatch.setattr(opool.PoolModel, "_release", release_always_free)
    assert _fails(*PREFIX_PINS) >= 1


# ---- stored tile orders ---------------------------------------------------------------------
def test_fp8_k_order_within_run_permutation_caught(monkeypatch):
    """Tokens of a 512-byte run nested [low][hi] instead of [hi][low]: a bijection that keeps
    every run contiguous, so only the hand-worked positions can tell it apart."""
    def k_offset_low_hi(t, d):
        return ((d // 64) * 2 + (t // 4) % 2) * 512 + ((t % 4) * 2 + t // 8) * 64 + d % 64

    monkeypatch.setattr(ofp8, "k_byte_offset", k_offset_low_hi)
    TF.test_k_layout_bijection_and_runs(128)  # the structural pins still pass
    assert _fails(TF.test_fp8_k_tile_order_fixture) == 1


def test_v_order_dimension_major_caught(monkeypatch):
    """The 16-bit V tile stored [D][16] (dimension rows of all 16 tokens) instead of
    [token half][D][8]."""
    def v_dim_major(self, blocks=slice(None)):
        v = self.v[blocks]
        return np.ascontiguousarray(v).reshape(v.shape[0], self.H, self.D * self.bs)

    monkeypatch.setattr(ocache.CacheModel, "v_physical", v_dim_major)
    assert _fails(TP.test_v_tile_order_fixture) == 1
