"""Block ids high enough that a tile's element and byte offsets pass 2^31 and 2^32 ([Serving]
"Production Serving: Continuous Batching and PagedAttention", Step 4: one tensor indexed by
physical page id, sized for the whole pool; a pool of 288 GB per GPU holds hundreds of thousands
of blocks).  A scene is built in a small pool, its tiles are copied into a large pool at an offset
past those bounds, and every entry point that addresses the cache (append, block copy, decode
single pass and split-K, grouped, allocation-free, fused append, prefill chunk, mixed launch;
bf16, fp32 and FP8 caches) must give bit for bit the same outputs and cache bytes as on the small
pool.  Only the addresses differ."""
import numpy as np
import pytest
import torch

import workloads as wl
from paged_kv_cache_404_amd import ops

from .gpu_util import Mirror, i32, to_dev
from .test_gpu_fp8 import Fp8Mirror

pytestmark = pytest.mark.gpu

# Block id from which (id * 8 heads * 16 tokens * 128 dims) elements exceed 2^31 (and bytes of a
# 2-byte type exceed 2^32).
OFF = (1 << 17) + 64
LENS = [700, 33, 1500, 16, 2049]
HQ, HKV, D = 32, 8, 128


def _big(small):
    big = torch.zeros((OFF + small.shape[0],) + tuple(small.shape[1:]), dtype=small.dtype, device="cuda")
    big[OFF:] = small
    return big


def _shift(tables):
    t = np.asarray(tables).copy()
    t[t >= 0] += OFF
    return t


def _eq(a, b):
    if a.dtype == torch.uint8:
        return torch.equal(a, b)
    return torch.equal(a.view(torch.int16 if a.element_size() == 2 else torch.int32),
                       b.view(torch.int16 if b.element_size() == 2 else torch.int32))


def _scene(make, dtype_in, seed):
    rng = np.random.default_rng(seed)
    need = sum(-(-L // 16) for L in LENS) + 16
    m = make(need, rng)
    seqs = [m.new_seq() for _ in LENS]
    tot = sum(LENS)
    m.append(seqs, LENS, wl.normal_bits(rng, (tot, HKV, D), dtype_in), wl.normal_bits(rng, (tot, HKV, D), dtype_in))
    return m, seqs, rng


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_large_block_ids(dtype):
    m, seqs, rng = _scene(lambda n, r: Mirror(n, HKV, D, dtype, r.permutation(n)), dtype, 3)
    tables, lens = m.tables(seqs)
    B, mcl, scale = len(LENS), int(lens.max()), 1 / np.sqrt(D)
    kb, vb = _big(m.k), _big(m.v)
    tb = _shift(tables)
    q = to_dev(wl.normal_bits(rng, (B, HQ, D), dtype), dtype)

    def both(fn):
        o_s = torch.full((B, HQ, D), float("nan"), device="cuda")
        o_b = torch.full_like(o_s, float("nan"))
        fn(o_s, m.k, m.v, i32(tables))
        fn(o_b, kb, vb, i32(tb))
        torch.cuda.synchronize()
        assert _eq(o_s, o_b)
        return o_s

    for ps in (0, 512):
        ws = ops.decode_workspace(B, HQ, D, mcl, ps)
        ref = both(lambda o, k, v, t: ops.paged_attention_decode(o, q, k, v, t, i32(lens), mcl, scale, ps, ws,
                                                                host_context_lens=lens))
        assert torch.isfinite(ref).all()
        if dtype == "bf16":
            g = both(lambda o, k, v, t: ops.paged_attention_decode_grouped(o, q, k, v, t, i32(lens), mcl, scale, 2,
                                                                          ps, ws))
            assert _eq(g, ref)
        if ps:
            n = both(lambda o, k, v, t: ops.paged_attention_decode_noalloc(o, q, k, v, t, i32(lens), mcl, scale, ps))
            assert _eq(n, ref)

    # prefill chunk: the last 100 cached tokens of sequence 2 as a chunk after 1,400
    C, ctx = 100, LENS[2] - 100
    qp = to_dev(wl.normal_bits(rng, (C, HQ, D), dtype), dtype)
    p_s = torch.full((C, HQ, D), float("nan"), device="cuda")
    p_b = torch.full_like(p_s, float("nan"))
    ops.paged_attention_prefill_chunk(p_s, qp, m.k, m.v, i32(tables[2]), ctx, scale)
    ops.paged_attention_prefill_chunk(p_b, qp, kb, vb, i32(tb[2]), ctx, scale)
    # mixed launch: every sequence's decode + that chunk
    d_s, d_b = torch.full_like(ref, float("nan")), torch.full_like(ref, float("nan"))
    x_s, x_b = torch.full_like(p_s, float("nan")), torch.full_like(p_s, float("nan"))
    ops.paged_attention_mixed(d_s, q, i32(tables), i32(lens), mcl, x_s, qp, i32(tables[2:3]), [ctx], [C], m.k, m.v,
                              scale)
    ops.paged_attention_mixed(d_b, q, i32(tb), i32(lens), mcl, x_b, qp, i32(tb[2:3]), [ctx], [C], kb, vb, scale)
    torch.cuda.synchronize()
    assert _eq(p_s, p_b) and torch.isfinite(p_s).all()
    assert _eq(d_s, d_b) and _eq(x_s, x_b)

    # one more token per sequence through the fused append, then 20 tokens of sequence 1 through
    # the append kernel, then a block copy
    st, _, slots, cow = m.pool.append_many(seqs, [1] * B)
    assert st == 0 and len(cow) == 0
    t2, l2 = m.pool.block_tables(seqs, tables.shape[1] + 1)
    nk = to_dev(wl.normal_bits(rng, (B, HKV, D), dtype), dtype)
    nv = to_dev(wl.normal_bits(rng, (B, HKV, D), dtype), dtype)
    ws = ops.decode_workspace(B, HQ, D, int(l2.max()), 512)
    f_s, f_b = torch.full_like(ref, float("nan")), torch.full_like(ref, float("nan"))
    ops.paged_attention_decode_append(f_s, q, nk, nv, m.k, m.v, i32(t2), i32(l2), int(l2.max()), scale, 512, ws)
    ops.paged_attention_decode_append(f_b, q, nk, nv, kb, vb, i32(_shift(t2)), i32(l2), int(l2.max()), scale, 512, ws)
    st, _, slots, cow = m.pool.append_many([seqs[1]], [20])
    assert st == 0
    ak = to_dev(wl.normal_bits(rng, (20, HKV, D), dtype), dtype)
    av = to_dev(wl.normal_bits(rng, (20, HKV, D), dtype), dtype)
    ops.paged_cache_append(m.k, m.v, ak, av, i32(slots))
    ops.paged_cache_append(kb, vb, ak, av, i32(slots + OFF * 16))
    src, dst = int(t2[2][0]), int(t2[4][0])
    ops.paged_cache_copy_blocks(m.k, m.v, i32([[src, dst]]))
    ops.paged_cache_copy_blocks(kb, vb, i32([[src + OFF, dst + OFF]]))
    torch.cuda.synchronize()
    assert _eq(f_s, f_b) and torch.isfinite(f_s).all()
    assert _eq(m.k, kb[OFF:]) and _eq(m.v, vb[OFF:])
    del kb, vb
    torch.cuda.empty_cache()


def test_large_block_ids_fp8():
    m, seqs, rng = _scene(lambda n, r: Fp8Mirror(n, HKV, D, r.permutation(n)), "bf16", 4)
    tables, lens = m.tables(seqs)
    B, mcl, scale = len(LENS), int(lens.max()), 1 / np.sqrt(D)
    kb, vb, ksb, vsb = _big(m.k), _big(m.v), _big(m.ks), _big(m.vs)
    tb = _shift(tables)
    q = to_dev(wl.normal_bits(rng, (B, HQ, D), "bf16"), "bf16")

    def both(fn):
        o_s = torch.full((B, HQ, D), float("nan"), device="cuda")
        o_b = torch.full_like(o_s, float("nan"))
        fn(o_s, m.k, m.v, m.ks, m.vs, i32(tables))
        fn(o_b, kb, vb, ksb, vsb, i32(tb))
        torch.cuda.synchronize()
        assert _eq(o_s, o_b)
        return o_s

    for ps in (0, 512):
        ws = ops.decode_workspace(B, HQ, D, mcl, ps)
        ref = both(lambda o, k, v, ks, vs, t: ops.paged_attention_decode_fp8(o, q, k, v, ks, vs, t, i32(lens), mcl,
                                                                            scale, ps, ws, host_context_lens=lens))
        assert torch.isfinite(ref).all()
        g = both(lambda o, k, v, ks, vs, t: ops.paged_attention_decode_grouped_fp8(o, q, k, v, ks, vs, t, i32(lens),
                                                                                  mcl, scale, 2, ps, ws))
        assert _eq(g, ref)

    C, ctx = 100, LENS[2] - 100
    qp = to_dev(wl.normal_bits(rng, (C, HQ, D), "bf16"), "bf16")
    p_s = torch.full((C, HQ, D), float("nan"), device="cuda")
    p_b = torch.full_like(p_s, float("nan"))
    ops.paged_attention_prefill_chunk_fp8(p_s, qp, m.k, m.v, m.ks, m.vs, i32(tables[2]), ctx, scale)
    ops.paged_attention_prefill_chunk_fp8(p_b, qp, kb, vb, ksb, vsb, i32(tb[2]), ctx, scale)
    d_s, d_b = torch.full_like(ref, float("nan")), torch.full_like(ref, float("nan"))
    x_s, x_b = torch.full_like(p_s, float("nan")), torch.full_like(p_s, float("nan"))
    ops.paged_attention_mixed_fp8(d_s, q, i32(tables), i32(lens), mcl, x_s, qp, i32(tables[2:3]), [ctx], [C], m.k,
                                  m.v, m.ks, m.vs, scale)
    ops.paged_attention_mixed_fp8(d_b, q, i32(tb), i32(lens), mcl, x_b, qp, i32(tb[2:3]), [ctx], [C], kb, vb, ksb,
                                  vsb, scale)
    torch.cuda.synchronize()
    assert _eq(p_s, p_b) and torch.isfinite(p_s).all()
    assert _eq(d_s, d_b) and _eq(x_s, x_b)

    st, _, slots, cow = m.pool.append_many(seqs, [1] * B)
    assert st == 0 and len(cow) == 0
    t2, l2 = m.pool.block_tables(seqs, tables.shape[1] + 1)
    nk = to_dev(wl.normal_bits(rng, (B, HKV, D), "bf16"), "bf16")
    nv = to_dev(wl.normal_bits(rng, (B, HKV, D), "bf16"), "bf16")
    f_s, f_b = torch.full_like(ref, float("nan")), torch.full_like(ref, float("nan"))
    ops.paged_attention_decode_append_fp8(f_s, q, nk, nv, m.k, m.v, m.ks, m.vs, i32(t2), i32(l2), int(l2.max()),
                                          scale)
    ops.paged_attention_decode_append_fp8(f_b, q, nk, nv, kb, vb, ksb, vsb, i32(_shift(t2)), i32(l2),
                                          int(l2.max()), scale)
    st, _, slots, cow = m.pool.append_many([seqs[1]], [20])
    assert st == 0
    ak = to_dev(wl.normal_bits(rng, (20, HKV, D), "bf16"), "bf16")
    av = to_dev(wl.normal_bits(rng, (20, HKV, D), "bf16"), "bf16")
    ops.paged_cache_append_fp8(m.k, m.v, m.ks, m.vs, ak, av, i32(slots))
    ops.paged_cache_append_fp8(kb, vb, ksb, vsb, ak, av, i32(slots + OFF * 16))
    src, dst = int(t2[2][0]), int(t2[4][0])
    ops.paged_cache_copy_blocks_fp8(m.k, m.v, m.ks, m.vs, i32([[src, dst]]))
    ops.paged_cache_copy_blocks_fp8(kb, vb, ksb, vsb, i32([[src + OFF, dst + OFF]]))
    torch.cuda.synchronize()
    assert _eq(f_s, f_b) and torch.isfinite(f_s).all()
    assert _eq(m.k, kb[OFF:]) and _eq(m.v, vb[OFF:])
    assert torch.equal(m.ks.view(torch.int32), ksb[OFF:].view(torch.int32))
    assert torch.equal(m.vs.view(torch.int32), vsb[OFF:].view(torch.int32))
    del kb, vb, ksb, vsb
    torch.cuda.empty_cache()
