"""Pins for the oracle's block pool and cache model (CPU).

Each test checks the oracle against something other than itself: the worked numbers in
tests/golden/ (derived by hand from the pages), closed forms, and invariants that hold for
any operation sequence.
"""
import json
import os

import numpy as np
import pytest

from oracle import CacheModel, InvalidOp, OutOfBlocks, PoolModel

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_alloc_pops_from_end_of_free_list():
    # Serving, Step 4: the free list starts as every id and alloc takes the last one.
    p = PoolModel(5)
    s = p.new_seq()
    slots, _ = p.append(s, 1)
    assert p.tables[s] == [4]
    assert slots == [4 * 16]
    p.append(s, 16)
    assert p.tables[s] == [4, 3]


def test_free_returns_blocks_in_table_order():
    # Serving, Step 4: finishing walks the page table in order and pushes each page back.
    p = PoolModel(6, free_order=[0, 1, 2, 3, 4, 5])
    s = p.new_seq()
    p.append(s, 40)  # blocks 5, 4, 3
    assert p.tables[s] == [5, 4, 3]
    p.free_seq(s)
    assert p.free == [0, 1, 2, 5, 4, 3]
    t = p.new_seq()
    p.append(t, 1)
    assert p.tables[t] == [3]  # the last page pushed is the first handed out again


def test_tiny_step_worked_tables():
    g = _golden("pool_worked_examples.json")["tiny_step_tables"]
    rng = np.random.default_rng(1)
    P = rng.permutation(32)
    pool = PoolModel(32, free_order=P)
    seqs = [pool.new_seq() for _ in g["lens"]]
    for s, L in zip(seqs, g["lens"]):
        pool.append(s, L - 1)
    step = [pool.append(s, 1)[0][0] for s in seqs]
    tables, lens = pool.block_tables(seqs, 3)
    want = [[int(P[i]) for i in row] for row in g["tables_as_free_order_index"]]
    assert [[b for b in r if b >= 0] for r in tables] == want
    assert lens == g["lens"]
    assert pool.num_free() == g["free_after"]
    assert step == [int(P[i]) * 16 + off for i, off in g["step_slots_as_index_and_offset"]]


def test_contiguous_vs_paged_accounting():
    g = _golden("pool_worked_examples.json")["contiguous_vs_paged"]
    assert g["requests"] * g["max_len"] == g["reserved_tokens_contiguous"]
    pool = PoolModel(2000)
    for _ in range(g["requests"]):
        s = pool.new_seq()
        pool.append(s, g["mean_len"])
    stored = sum(pool.lens.values())
    allocated = (2000 - pool.num_free()) * 16
    assert stored == g["stored_tokens"]
    assert stored / g["reserved_tokens_contiguous"] == g["fraction_used_contiguous"]
    assert abs(g["fraction_used_contiguous"] - g["page_fraction_used_printed"]) < 0.0013
    assert allocated == g["paged_slots_allocated_when_every_len_is_200"]


def test_tail_waste_bound_is_block_size_minus_one():
    g = _golden("pool_worked_examples.json")["tail_waste_bound"]
    worst = 0
    for L in range(1, 200):
        pool = PoolModel(20)
        s = pool.new_seq()
        pool.append(s, L)
        waste = len(pool.tables[s]) * 16 - L
        worst = max(worst, waste)
        assert waste == (-L) % 16
        if L % 16 == 1:
            assert waste == g["max_waste_per_sequence"]
    assert worst == g["max_waste_per_sequence"]
    assert 100 * worst == g["max_waste_per_100_sequences"]


def test_reserve_32k_use_2k():
    g = _golden("pool_worked_examples.json")["reserve_32k_use_2k"]
    assert 1 - g["used"] / g["reserved"] == g["fraction_empty"]
    pool = PoolModel(200)
    s = pool.new_seq()
    pool.append(s, g["used"])
    assert len(pool.tables[s]) == g["paged_blocks"]
    assert len(pool.tables[s]) * 16 - g["used"] == g["paged_waste"]


def test_out_of_blocks_is_all_or_nothing():
    pool = PoolModel(3)
    a = pool.new_seq()
    pool.append(a, 20)  # 2 blocks
    b = pool.new_seq()
    before = (list(pool.free), list(pool.refcnt), {k: list(v) for k, v in pool.tables.items()}, dict(pool.lens))
    with pytest.raises(OutOfBlocks):
        pool.append(b, 17)  # needs 2, one free
    after = (list(pool.free), list(pool.refcnt), {k: list(v) for k, v in pool.tables.items()}, dict(pool.lens))
    assert before == after
    pool.append(b, 16)  # exactly one block fits
    with pytest.raises(OutOfBlocks):
        pool.append(b, 1)


def test_fork_shares_and_cow_isolates():
    pool = PoolModel(10, free_order=list(range(10)))
    p = pool.new_seq()
    pool.append(p, 20)  # blocks 9 (full) and 8 (4 tokens)
    c = pool.fork(p)
    assert pool.tables[c] == [9, 8] and pool.refcnt[9] == 2 and pool.refcnt[8] == 2
    slots, cow = pool.append(c, 1)
    assert cow == [(8, 7)]
    assert pool.tables[c] == [9, 7] and pool.tables[p] == [9, 8]
    assert slots == [7 * 16 + 4]
    assert pool.refcnt[8] == 1 and pool.refcnt[7] == 1 and pool.refcnt[9] == 2
    # the parent now owns its partial block alone and writes in place
    slots, cow = pool.append(p, 1)
    assert cow == [] and slots == [8 * 16 + 4]


def test_fork_on_block_boundary_never_copies():
    pool = PoolModel(8)
    p = pool.new_seq()
    pool.append(p, 32)
    c = pool.fork(p)
    slots, cow = pool.append(c, 1)
    assert cow == [] and len(pool.tables[c]) == 3 and pool.tables[c][:2] == pool.tables[p]


def test_sixteen_samples_on_partial_prefix():
    # 2,040-token prefix (last block 8/16 full) forked to 16 samples; appending in batch order,
    # samples 0..14 copy the shared block and the last one finds refcount 1 and writes in place.
    pool = PoolModel(200)
    s0 = pool.new_seq()
    pool.append(s0, 2040)
    samples = [s0] + [pool.fork(s0) for _ in range(15)]
    shared_last = pool.tables[s0][-1]
    assert pool.refcnt[shared_last] == 16
    cows = [pool.append(s, 1)[1] for s in samples]
    assert all(len(c) == 1 and c[0][0] == shared_last for c in cows[:15])
    assert cows[15] == []
    assert pool.tables[samples[15]][-1] == shared_last
    assert pool.refcnt[shared_last] == 1


def test_blocks_needed_matches_append():
    rng = np.random.default_rng(7)
    pool = PoolModel(400, free_order=rng.permutation(400))
    seqs = [pool.new_seq() for _ in range(4)]
    for _ in range(200):
        s = seqs[rng.integers(len(seqs))]
        n = int(rng.integers(0, 40))
        need = pool.blocks_needed(s, n)
        free0 = pool.num_free()
        try:
            pool.append(s, n)
            assert free0 - pool.num_free() == need
        except OutOfBlocks:
            assert need > free0
        if rng.random() < 0.2:
            seqs.append(pool.fork(s))
        if rng.random() < 0.1 and len(seqs) > 1:
            v = seqs.pop(int(rng.integers(len(seqs))))
            pool.free_seq(v)


def _check_invariants(pool):
    N = pool.num_blocks
    free = pool.free
    assert len(set(free)) == len(free)
    held = set()
    ref = [0] * N
    for t in pool.tables.values():
        for b in t:
            ref[b] += 1
            held.add(b)
    assert held.isdisjoint(free)
    assert held | set(free) == set(range(N))
    assert ref == pool.refcnt
    for s, t in pool.tables.items():
        assert len(t) == -(-pool.lens[s] // pool.block_size)


def test_random_operation_invariants():
    rng = np.random.default_rng(11)
    pool = PoolModel(64, free_order=rng.permutation(64))
    live = []
    for step in range(3000):
        r = rng.random()
        if r < 0.15 or not live:
            live.append(pool.new_seq())
        elif r < 0.25:
            live.append(pool.fork(live[int(rng.integers(len(live)))]))
        elif r < 0.40:
            pool.free_seq(live.pop(int(rng.integers(len(live)))))
        else:
            s = live[int(rng.integers(len(live)))]
            try:
                _, cow = pool.append(s, int(rng.integers(1, 24)))
                for old, new in cow:
                    assert pool.refcnt[new] == 1
            except OutOfBlocks:
                pass
        _check_invariants(pool)
    for s in list(live):
        pool.free_seq(s)
    assert sorted(pool.free) == list(range(64))
    assert all(c == 0 for c in pool.refcnt)


def test_sequence_ids_lowest_free():
    pool = PoolModel(4)
    a, b, c = pool.new_seq(), pool.new_seq(), pool.new_seq()
    assert (a, b, c) == (0, 1, 2)
    pool.free_seq(b)
    assert pool.new_seq() == 1
    assert pool.fork(a) == 3


def test_invalid_ops():
    pool = PoolModel(4)
    with pytest.raises(InvalidOp):
        pool.append(5, 1)
    with pytest.raises(InvalidOp):
        pool.free_seq(0)
    with pytest.raises(InvalidOp):
        PoolModel(3, free_order=[0, 0, 1])
    s = pool.new_seq()
    pool.append(s, 3)
    with pytest.raises(InvalidOp):
        pool.block_tables([s], 0)


def test_cache_layout_fixture():
    g = _golden("cache_layout.json")
    c = CacheModel(g["num_blocks"], g["num_kv_heads"], g["head_dim"], "f32", g["block_size"], fill_nan=True)
    keys = np.array([t["k"] for t in g["tokens"]], dtype=np.float32).view(np.uint32)
    vals = np.array([t["v"] for t in g["tokens"]], dtype=np.float32).view(np.uint32)
    c.append(keys, vals, [t["slot"] for t in g["tokens"]])
    kf, vf = c.k.view(np.float32), c.v.view(np.float32)
    for e in g["expect_k"]:
        assert kf[tuple(e["index"])] == e["value"]
    for e in g["expect_v"]:
        assert vf[tuple(e["index"])] == e["value"]
    assert (~np.isnan(kf)).sum() == g["written_elements_per_tensor"]
    assert (~np.isnan(vf)).sum() == g["written_elements_per_tensor"]
    assert not (kf == 99).any() and not (vf == 99).any()


def test_copy_blocks_whole_block():
    rng = np.random.default_rng(3)
    c = CacheModel(4, 2, 8, "bf16")
    c.k[1] = rng.integers(0, 1 << 16, size=c.k[1].shape, dtype=np.uint16)
    c.v[1] = rng.integers(0, 1 << 16, size=c.v[1].shape, dtype=np.uint16)
    k1, v1, k2 = c.k[1].copy(), c.v[1].copy(), c.k[2].copy()
    c.copy_blocks([(1, 3)])
    assert (c.k[3] == k1).all() and (c.v[3] == v1).all()
    assert (c.k[1] == k1).all() and (c.k[2] == k2).all()


def test_k_tile_order_fixture():
    """Single elements land where the hand-worked fixture puts them."""
    for case in _golden("k_tile_order.json")["cases"]:
        dt, D = case["dtype"], case["head_dim"]
        c = CacheModel(2, 2, D, dt, fill_nan=False)
        c.k[1, 1, case["token"], case["dim"]] = 7
        phys = c.k_physical()
        assert phys[1, 1, case["element_offset"]] == 7, case
        assert np.count_nonzero(phys) == 1


@pytest.mark.parametrize("dt,D", [("bf16", 128), ("bf16", 64), ("f16", 128), ("f32", 64), ("f32", 128)])
def test_k_tile_order_is_a_permutation_with_contiguous_k_steps(dt, D):
    """Every element appears once; and, the point of the order, the 8 tokens of one token set
    times the 4 chunks of one 32-byte-per-chunk-group k-step occupy one contiguous run of 32
    chunks (512 bytes for 16-bit types)."""
    c = CacheModel(1, 1, D, dt, fill_nan=False)
    E = 16 // c.k.dtype.itemsize
    ids = np.arange(16 * D).reshape(16, D)  # logical id = t * D + d (fits the storage type)
    c.k[0, 0] = ids
    phys = c.k_physical()[0, 0].astype(np.int64)
    assert sorted(phys.tolist()) == list(range(16 * D))
    chunks = phys.reshape(-1, E)
    assert (chunks == chunks[:, :1] + np.arange(E)).all()  # a chunk keeps its elements in order
    tok = chunks[:, 0] // D
    cidx = (chunks[:, 0] % D) // E
    for run in range(len(chunks) // 32):
        t, ch = tok[run * 32:(run + 1) * 32], cidx[run * 32:(run + 1) * 32]
        assert len(set((t // 4) % 2)) == 1 and len(set(ch // 4)) == 1  # one token set, one chunk group
        assert sorted(zip(t.tolist(), ch.tolist())) == sorted(
            (tt, cq * 4 + cr) for tt in range(16) if (tt // 4) % 2 == (t[0] // 4) % 2
            for cq in [ch[0] // 4] for cr in range(4))


# ---- prefix cache ([Serving] The Build, Step 8), values worked by hand ----------------------

T40 = list(range(100, 140))


def test_prefix_cache_worked_scenario():
    p = PoolModel(8, 16)  # free list 0..7: allocation takes 7, 6, 5, ...
    s0 = p.new_seq()
    p.append(s0, 40)
    assert p.tables[s0] == [7, 6, 5]
    assert p.prefix_insert(s0, T40) == 2  # two full blocks: prefixes of 16 and 32 tokens
    assert p.entries == {tuple(T40[:16]): [7], tuple(T40[:32]): [7, 6]}
    s1, n = p.prefix_lookup(T40)  # longest block-aligned match: 32 tokens (40 is not aligned)
    assert (s1, n, p.tables[s1], p.lens[s1]) == (1, 32, [7, 6], 32)
    assert p.refcnt[7] == 2 and p.refcnt[6] == 2
    s2, n = p.prefix_lookup(T40[:20] + [999] * 20)  # diverges inside the second block
    assert (s2, n, p.tables[s2]) == (2, 16, [7])
    s3, n = p.prefix_lookup([5] + T40[1:])  # diverges in the first token
    assert (s3, n, p.tables[s3]) == (3, 0, [])
    assert p.refcnt[7] == 3
    p.free_seq(s0)  # 7: 3 -> 2, 6: 2 -> 1, 5: 1 -> 0 and unregistered -> free list
    assert p.free == [0, 1, 2, 3, 4, 5] and p.lru == []
    p.free_seq(s1)  # 7: 2 -> 1, 6: 1 -> 0, registered -> LRU
    p.free_seq(s2)  # 7: 1 -> 0 -> LRU behind 6
    p.free_seq(s3)
    assert p.lru == [6, 7] and p.free == [0, 1, 2, 3, 4, 5]
    s, n = p.prefix_lookup(T40)  # a hit on unreferenced blocks takes them off the LRU
    assert (s, n, p.tables[s], p.lru) == (0, 32, [7, 6], [])
    p.free_seq(s)  # both reach zero together: they join the LRU deepest first
    assert p.lru == [6, 7]
    s = p.new_seq()
    p.append(s, 96)  # the six free blocks, last first
    assert p.tables[s] == [5, 4, 3, 2, 1, 0] and p.free == []
    p.append(s, 1)  # free list empty: evict the LRU head (6), which only the 32-token prefix uses
    assert p.tables[s] == [5, 4, 3, 2, 1, 0, 6]
    assert p.entries == {tuple(T40[:16]): [7]} and p.lru == [7] and p.free == []
    s4, n = p.prefix_lookup(T40)
    assert n == 16 and p.tables[s4] == [7] and p.lru == []
    p.append(s, 15)  # fills block 6 (positions 97..111): the next token needs a block, none is left
    with pytest.raises(OutOfBlocks):
        p.append(s, 1)
    p.free_seq(s4)
    p.append(s, 1)  # now 7 is evictable: the last registered prefix goes
    assert p.tables[s][-1] == 7 and p.entries == {} and p.lru == []


def test_prefix_cache_shares_the_common_first_block():
    p = PoolModel(8, 16)
    a = [1] * 16 + [2] * 16
    b = [1] * 16 + [3] * 16
    s0, s1 = p.new_seq(), p.new_seq()
    p.append(s0, 32)
    p.append(s1, 32)
    assert p.tables[s0] == [7, 6] and p.tables[s1] == [5, 4]
    assert p.prefix_insert(s0, a) == 2
    assert p.prefix_insert(s1, b) == 1  # the 16-token prefix is already held by block 7
    assert p.entries[tuple(b)] == [7, 4]
    assert p.prefix_insert(s1, b) == 0  # registering again changes nothing
    s, n = p.prefix_lookup(b + [9] * 5)
    assert (n, p.tables[s]) == (32, [7, 4])
    s2, n = p.prefix_lookup(a)  # the whole request may match
    assert (n, p.tables[s2]) == (32, [7, 6])
    p.free_seq(s1)  # 5 was never registered (a duplicate of 7's tokens): straight to the free list
    assert p.free[-1] == 5 and p.refcnt[4] == 1 and p.lru == []
    # a block registered under one prefix is not registered under another
    assert p.prefix_insert(s0, [8] * 32) == 0


def test_prefix_cache_capacity_counts_the_lru():
    p = PoolModel(4, 16)
    s = p.new_seq()
    p.append(s, 64)
    toks = list(range(64))
    assert p.prefix_insert(s, toks) == 4
    p.free_seq(s)
    assert p.free == [] and p.lru == [0, 1, 2, 3]  # deepest block first
    t = p.new_seq()
    with pytest.raises(OutOfBlocks):
        p.append(t, 65)  # five blocks > 0 free + 4 evictable
    assert p.lru == [0, 1, 2, 3] and p.tables[t] == []  # all-or-nothing
    p.append(t, 17)  # two blocks: the two deepest registered blocks are evicted
    assert p.tables[t] == [0, 1] and p.free == [] and p.lru == [2, 3]
    assert p.entries == {tuple(toks[:16]): [3], tuple(toks[:32]): [3, 2]}
    p.free_seq(t)  # 0 and 1 are no longer registered: straight to the free list
    assert p.free == [0, 1] and p.lru == [2, 3]
    p.append(p.new_seq(), 64)  # free blocks first (1, 0), then the LRU: 2, then 3 (its child gone)
    assert p.entries == {} and p.lru == [] and p.free == []


def test_prefix_cache_random_invariants():
    rng = np.random.default_rng(11)
    p = PoolModel(24, 16, rng.permutation(24))
    live, toks = [], {}
    for _ in range(400):
        r = rng.random()
        if r < 0.2 or not live:
            t = [int(x) for x in rng.integers(0, 2, int(rng.integers(0, 80)))]
            s, n = p.prefix_lookup(t)
            # the match is the longest registered aligned prefix: no longer one is registered
            assert n % 16 == 0 and tuple(t[:n]) in p.entries or n == 0
            assert all(tuple(t[:m]) not in p.entries for m in range(n + 16, len(t) // 16 * 16 + 1, 16))
            live.append(s)
            toks[s] = t[:n]
        elif r < 0.35:
            s = live.pop(int(rng.integers(len(live))))
            p.free_seq(s)
            del toks[s]
        elif r < 0.5:
            s = live[int(rng.integers(len(live)))]
            p.prefix_insert(s, toks[s])
        else:
            s = live[int(rng.integers(len(live)))]
            n = int(rng.integers(0, 30))
            try:
                p.append(s, n)
            except OutOfBlocks:
                continue
            toks[s] = toks[s] + [int(x) for x in rng.integers(0, 2, n)]
        # every block is in exactly one of: referenced, free list, LRU
        held = {b for b in range(24) if p.refcnt[b] > 0}
        assert len(held) + len(p.free) + len(p.lru) == 24
        assert not (held & set(p.free)) and not (held & set(p.lru)) and not (set(p.free) & set(p.lru))
        reg = {b for blocks in p.entries.values() for b in blocks}
        assert set(p.lru) <= reg and not (set(p.free) & reg)
        # every registered prefix's shorter aligned prefixes are registered, with the same blocks
        for key, blocks in p.entries.items():
            assert len(key) == 16 * len(blocks)
            if len(blocks) > 1:
                assert p.entries[key[:-16]] == blocks[:-1]


def test_prefix_cache_eviction_unregisters_the_blocks_below():
    """A block registered below another sequence's block: evicting the parent must unregister it
    even though its own holder still references it."""
    p = PoolModel(6, 16)  # allocation takes 5, 4, 3, ...
    x, y = p.new_seq(), p.new_seq()
    p.append(x, 16)
    p.append(y, 32)
    assert p.tables[x] == [5] and p.tables[y] == [4, 3]
    a = [1] * 16
    b = a + [2] * 16
    assert p.prefix_insert(x, a) == 1
    assert p.prefix_insert(y, b) == 1  # the 16-token prefix is block 5; y's block 3 goes below it
    assert p.entries == {tuple(a): [5], tuple(b): [5, 3]}
    p.free_seq(x)  # 5 reaches zero while 3, below it, is still held by y
    assert p.lru == [5] and p.free == [0, 1, 2]
    z = p.new_seq()
    p.append(z, 48)  # 2, 1, 0
    p.append(z, 1)  # evicts 5: both prefixes go, and 3 is no longer registered
    assert p.tables[z] == [2, 1, 0, 5] and p.entries == {} and p.lru == []
    s, n = p.prefix_lookup(b)
    assert n == 0
    p.free_seq(y)  # 4 and 3 are unregistered: both to the free list
    assert p.free == [4, 3] and p.lru == []


@pytest.mark.parametrize("dt,D", [("bf16", 128), ("f32", 64), ("f16", 64)])
def test_v_tile_order_by_brute_force(dt, D):
    """The stored V order, element by element: (block, head, dimension d, token t) sits at
    ((t // 8) * D + d) * 8 + t % 8 of its tile; 16 dimensions of one 8-token half are 256
    contiguous bytes at 16-bit elements (one half-wave operand load)."""
    rng = np.random.default_rng(7)
    N, H = 3, 2
    cache = CacheModel(N, H, D, dt, fill_nan=False)
    cache.v[:] = rng.integers(1, 2**15, size=cache.v.shape).astype(cache.v.dtype)
    phys = cache.v_physical()
    for b in range(N):
        for h in range(H):
            for d in range(D):
                for t in range(16):
                    assert phys[b, h, ((t // 8) * D + d) * 8 + t % 8] == cache.v[b, h, d, t]
    esize = cache.v.dtype.itemsize
    if esize == 2:
        # a half-wave's 16 lanes (dimensions 16 nb .. 16 nb + 15 of one half) read 256 contiguous bytes
        assert (16 * 8 * esize) == 256


def test_v_tile_order_fixture():
    """Hand-worked element positions of the 16-bit and fp32 V tile ([token half][D][8 tokens]):
    a token appended with one marked element lands there in the stored order, and nowhere else."""
    for case in _golden("v_tile_order.json")["cases"]:
        dt = case["dtype"]
        if dt == "fp8":
            continue
        D, t, d, off = case["head_dim"], case["token"], case["dim"], case["element_offset"]
        c = CacheModel(2, 2, D, dt, fill_nan=False)
        row = np.zeros((1, 2, D), dtype=c.v.dtype)
        row[0, 1, d] = 5
        c.append(row, row, [16 + t])
        phys = c.v_physical()
        assert phys[1, 1, off] == 5, case
        assert np.count_nonzero(phys) == 1, case
