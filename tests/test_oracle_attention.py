"""Pins for the oracle's paged attention (CPU).

The pages print no attention value, so the fp64 oracle is pinned by: the pure-Python
brute force that walks the page table like the pages' loops; an independent library
routine (torch's scaled_dot_product_attention in fp64 on the CPU); closed forms
(one token returns V, a zero query averages V, constant V, two tokens give a logistic
weight, a huge scale picks the arg-max token); and invariants (weights sum to one,
physical-block permutation, GQA equals MHA on repeated K/V, block-size independence,
prefill row i equals a decode of length ctx_start + i + 1).
"""
import math

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import CacheModel, PoolModel, attention, brute


def _build(seed, lens, Hq, Hkv, D, dtype, bs=16, extra_blocks=3):
    rng = np.random.default_rng(seed)
    N = sum(-(-L // bs) for L in lens) + extra_blocks
    pool = PoolModel(N, bs, free_order=rng.permutation(N))
    cache = CacheModel(N, Hkv, D, dtype, bs)
    seqs = []
    for L in lens:
        s = pool.new_seq()
        slots, _ = pool.append(s, L)
        k = wl.normal_bits(rng, (L, Hkv, D), dtype)
        v = wl.normal_bits(rng, (L, Hkv, D), dtype)
        cache.append(k, v, slots)
        seqs.append(s)
    q = wl.normal_bits(rng, (len(lens), Hq, D), dtype)
    tables, _ = pool.block_tables(seqs, max(-(-L // bs) for L in lens))
    return pool, cache, tables, q


@pytest.mark.parametrize("dtype,Hq,Hkv,D", [("f32", 2, 2, 4), ("bf16", 4, 1, 4), ("f16", 4, 2, 8), ("bf16", 8, 2, 4)])
def test_numpy_oracle_equals_brute_force(dtype, Hq, Hkv, D):
    lens = [1, 7, 16, 17, 40]
    pool, cache, tables, q = _build(5, lens, Hq, Hkv, D, dtype)
    scale = 1 / math.sqrt(D)
    out = attention.paged_decode(q, cache, tables, lens, scale)
    for b, L in enumerate(lens):
        table = [t for t in tables[b] if t >= 0]
        for h in range(Hq):
            ref, _ = brute.decode_one(q[b, h], cache, table, L, h, Hq, scale)
            np.testing.assert_allclose(out[b, h], ref, rtol=0, atol=1e-12)


def test_matches_torch_sdpa_fp64():
    lens = [3, 33, 64, 129]
    Hq, Hkv, D = 8, 2, 16
    pool, cache, tables, q = _build(9, lens, Hq, Hkv, D, "bf16")
    scale = 0.37
    out = attention.paged_decode(q, cache, tables, lens, scale)
    qf = attention.bits_to_f64(q, "bf16")
    for b, L in enumerate(lens):
        K, V = attention.gather(cache, tables[b], L)
        Kt = torch.from_numpy(np.repeat(K, Hq // Hkv, axis=0))[None]
        Vt = torch.from_numpy(np.repeat(V, Hq // Hkv, axis=0))[None]
        Qt = torch.from_numpy(qf[b])[None, :, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(Qt, Kt, Vt, scale=scale)[0, :, 0, :]
        np.testing.assert_allclose(out[b], ref.numpy(), rtol=0, atol=1e-12)


def test_gather_round_trip_recovers_tokens_in_order():
    rng = np.random.default_rng(2)
    pool = PoolModel(12, free_order=rng.permutation(12))
    cache = CacheModel(12, 3, 5, "f32")
    s = pool.new_seq()
    L = 37
    slots, _ = pool.append(s, L)
    k = np.arange(L * 15, dtype=np.float32).reshape(L, 3, 5)
    v = -k
    cache.append(k.view(np.uint32), v.view(np.uint32), slots)
    K, V = attention.gather(cache, pool.tables[s], L)
    np.testing.assert_array_equal(K, k.transpose(1, 0, 2))
    np.testing.assert_array_equal(V, v.transpose(1, 0, 2))


def test_single_token_returns_v_exactly():
    pool, cache, tables, q = _build(4, [1, 1], 4, 2, 8, "bf16")
    out = attention.paged_decode(q, cache, tables, [1, 1], 0.3)
    for b in range(2):
        K, V = attention.gather(cache, tables[b], 1)
        for h in range(4):
            assert (out[b, h] == V[h // 2, 0]).all()


def test_weights_sum_to_one_and_zero_query_averages():
    lens = [5, 50, 100]
    pool, cache, tables, q = _build(6, lens, 4, 4, 8, "f32")
    out, w = attention.paged_decode(q, cache, tables, lens, 0.5, return_weights=True)
    for (b, h), wt in w.items():
        assert abs(wt.sum() - 1) < 1e-12 and (wt > 0).all()
    q0 = np.zeros_like(q)
    out0 = attention.paged_decode(q0, cache, tables, lens, 0.5)
    for b, L in enumerate(lens):
        K, V = attention.gather(cache, tables[b], L)
        np.testing.assert_allclose(out0[b], V.mean(axis=1), rtol=0, atol=1e-12)


def test_constant_values_give_that_constant():
    lens = [9, 31]
    pool, cache, tables, q = _build(8, lens, 2, 2, 4, "f32")
    cache.v[:] = np.float32(1.25).view(np.uint32)
    out = attention.paged_decode(q, cache, tables, lens, 1.0)
    np.testing.assert_allclose(out, 1.25, rtol=0, atol=1e-14)


def test_two_token_closed_form():
    # q = (1, 0), k0 = (2, 0), k1 = (0, 0): scores (2, 0); weight of token 0 is the logistic of 2.
    cache = CacheModel(1, 1, 2, "f32")
    keys = np.array([[[2, 0]], [[0, 0]]], dtype=np.float32).view(np.uint32)
    vals = np.array([[[1, 2]], [[3, -1]]], dtype=np.float32).view(np.uint32)
    cache.append(keys, vals, [0, 1])
    q = np.array([[[1, 0]]], dtype=np.float32).view(np.uint32)
    out = attention.paged_decode(q, cache, [[0]], [2], 1.0)[0, 0]
    w0 = 1 / (1 + math.exp(-2))
    np.testing.assert_allclose(out, [w0 * 1 + (1 - w0) * 3, w0 * 2 + (1 - w0) * -1], rtol=0, atol=1e-15)


def test_huge_scale_selects_argmax_token():
    lens = [40]
    pool, cache, tables, q = _build(12, lens, 2, 1, 8, "f32")
    K, V = attention.gather(cache, tables[0], 40)
    qf = attention.bits_to_f64(q, "f32")
    out = attention.paged_decode(q, cache, tables, lens, 1e4)
    for h in range(2):
        t = int(np.argmax(K[0] @ qf[0, h]))
        np.testing.assert_allclose(out[0, h], V[0, t], rtol=0, atol=1e-9)


def test_physical_block_permutation_invariance():
    lens = [20, 45]
    pool, cache, tables, q = _build(13, lens, 4, 2, 8, "bf16", extra_blocks=0)
    out = attention.paged_decode(q, cache, tables, lens, 0.35)
    N = cache.N
    perm = np.random.default_rng(0).permutation(N)  # old block b moves to perm[b]
    moved = CacheModel(N, cache.H, cache.D, "bf16")
    moved.k[perm] = cache.k
    moved.v[perm] = cache.v
    new_tables = [[int(perm[b]) if b >= 0 else -1 for b in row] for row in tables]
    out2 = attention.paged_decode(q, moved, new_tables, lens, 0.35)
    assert (out == out2).all()


def test_gqa_equals_mha_on_repeated_kv():
    lens = [18, 33]
    Hq, Hkv, D = 8, 2, 8
    pool, cache, tables, q = _build(14, lens, Hq, Hkv, D, "bf16")
    out = attention.paged_decode(q, cache, tables, lens, 0.3)
    G = Hq // Hkv
    rep = CacheModel(cache.N, Hq, D, "bf16")
    rep.k = np.repeat(cache.k, G, axis=1)
    rep.v = np.repeat(cache.v, G, axis=1)
    out_mha = attention.paged_decode(q, rep, tables, lens, 0.3)
    assert (out == out_mha).all()


def test_block_size_independence():
    rng = np.random.default_rng(15)
    L, H, D = 50, 2, 4
    k = wl.normal_bits(rng, (L, H, D), "bf16")
    v = wl.normal_bits(rng, (L, H, D), "bf16")
    q = wl.normal_bits(rng, (1, 4, D), "bf16")
    outs = []
    for bs in (16, 1, 7, L):
        nb = -(-L // bs)
        pool = PoolModel(nb + 2, bs, free_order=rng.permutation(nb + 2))
        cache = CacheModel(nb + 2, H, D, "bf16", bs)
        s = pool.new_seq()
        slots, _ = pool.append(s, L)
        cache.append(k, v, slots)
        outs.append(attention.paged_decode(q, cache, [pool.tables[s]], [L], 0.5))
    for o in outs[1:]:
        np.testing.assert_allclose(o, outs[0], rtol=0, atol=1e-13)


def test_prefill_rows_equal_decodes_and_sdpa_causal():
    rng = np.random.default_rng(16)
    ctx, C, Hq, Hkv, D = 21, 12, 4, 2, 8
    total = ctx + C
    pool = PoolModel(6, free_order=rng.permutation(6))
    cache = CacheModel(6, Hkv, D, "bf16")
    s = pool.new_seq()
    slots, _ = pool.append(s, total)
    cache.append(wl.normal_bits(rng, (total, Hkv, D), "bf16"), wl.normal_bits(rng, (total, Hkv, D), "bf16"), slots)
    q = wl.normal_bits(rng, (C, Hq, D), "bf16")
    table = pool.tables[s]
    out = attention.prefill_chunk(q, cache, table, ctx, 0.4)
    for i in range(C):
        dec = attention.paged_decode(q[i:i + 1], cache, [table], [ctx + i + 1], 0.4)
        np.testing.assert_allclose(out[i], dec[0], rtol=0, atol=1e-13)
    K, V = attention.gather(cache, table, total)
    qf = attention.bits_to_f64(q, "bf16")
    mask = np.arange(total)[None, :] <= (ctx + np.arange(C))[:, None]
    Qt = torch.from_numpy(qf.transpose(1, 0, 2))[None]
    Kt = torch.from_numpy(np.repeat(K, 2, axis=0))[None]
    Vt = torch.from_numpy(np.repeat(V, 2, axis=0))[None]
    ref = torch.nn.functional.scaled_dot_product_attention(Qt, Kt, Vt, attn_mask=torch.from_numpy(mask), scale=0.4)
    np.testing.assert_allclose(out, ref[0].numpy().transpose(1, 0, 2), rtol=0, atol=1e-12)


def test_prefill_first_row_of_empty_context_returns_v():
    rng = np.random.default_rng(17)
    pool = PoolModel(3)
    cache = CacheModel(3, 1, 4, "f32")
    s = pool.new_seq()
    slots, _ = pool.append(s, 5)
    v = wl.normal_bits(rng, (5, 1, 4), "f32")
    cache.append(wl.normal_bits(rng, (5, 1, 4), "f32"), v, slots)
    out = attention.prefill_chunk(wl.normal_bits(rng, (5, 2, 4), "f32"), cache, pool.tables[s], 0, 0.5)
    assert (out[0, 0] == v[0, 0].view(np.float32)).all() and (out[0, 1] == v[0, 0].view(np.float32)).all()


def test_stale_tail_slots_are_never_read():
    # Cache prefilled with NaN: only stored tokens may take part.
    lens = [3, 17]
    pool, cache, tables, q = _build(18, lens, 2, 2, 4, "bf16")
    out = attention.paged_decode(q, cache, tables, lens, 0.5)
    assert np.isfinite(out).all()
