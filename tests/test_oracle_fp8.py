"""Pins of the FP8 (OCP E4M3) cache oracle (CPU only).

The codec is pinned to values the OCP 8-bit floating point format fixes (named codes, the
largest finite value, the NaN codes, the subnormal step), to a round trip over every code, and
to a brute-force nearest-even search over the whole code table; the quantisation to its error
bounds and special cases; the tile layout to being a bijection with the contiguity the kernels
rely on."""
import json
import os

import numpy as np
import pytest

from oracle import Fp8CacheModel
from oracle import attention as oatt
from oracle import fp8

FINITE = [c for c in range(256) if (c & 0x7F) != 0x7F]


def test_named_codes():
    d = fp8.e4m3_decode
    assert d(0x00) == 0.0 and np.signbit(d(0x80))
    assert d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9  # subnormals: m * 2^-9
    assert d(0x08) == 2.0 ** -6  # smallest normal
    assert d(0x38) == 1.0 and d(0x3A) == 1.25 and d(0x40) == 2.0 and d(0xB8) == -1.0
    assert d(0x77) == 240.0 and d(0x7E) == 448.0 and d(0xFE) == -448.0  # largest finite
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))  # the only NaNs; no infinities


def test_round_trip_every_code():
    codes = np.array(FINITE)
    assert np.array_equal(fp8.e4m3_encode(fp8.e4m3_decode(codes)), codes.astype(np.uint8))


def test_encode_is_nearest_even_by_brute_force():
    rng = np.random.default_rng(3)
    vals = np.concatenate([rng.uniform(-463.9, 463.9, 4000), rng.uniform(-0.05, 0.05, 4000),
                           rng.uniform(-2.0 ** -6, 2.0 ** -6, 2000)]).astype(np.float32).astype(np.float64)
    table = fp8.e4m3_decode(np.array(FINITE))
    got = fp8.e4m3_encode(vals)
    for x, c in zip(vals, got):
        dist = np.abs(table - x)
        best = np.flatnonzero(dist == dist.min())
        cand = [FINITE[i] for i in best]
        if len(cand) > 1:  # a tie: the even code (ignoring +0 / -0 duplicates)
            vals_c = {float(fp8.e4m3_decode(c)) for c in cand}
            if len(vals_c) > 1:
                cand = [c for c in cand if c % 2 == 0]
        assert int(c) in cand or (x == 0.0), (x, c, cand)


def test_ties_and_bounds():
    e = fp8.e4m3_encode
    assert e(1.0625) == 0x38 and e(1.1875) == 0x3A  # halfway cases go to the even mantissa
    assert e(1.5 * 2.0 ** -9) == 0x02 and e(2.5 * 2.0 ** -9) == 0x02 and e(0.5 * 2.0 ** -9) == 0x00
    assert e(448.0 * (1 + 2.0 ** -23)) == 0x7E and e(463.9) == 0x7E
    assert e(-0.0) == 0x80
    with pytest.raises(ValueError):
        e(464.0)


def test_quantize_rows_error_bound_and_specials():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((200, 128)) * rng.uniform(1e-3, 50.0, (200, 1))).astype(np.float32)
    codes, s = fp8.quantize_rows(x)
    deq = fp8.e4m3_decode(codes) * s[:, None].astype(np.float64)
    amax = np.abs(x).max(axis=1).astype(np.float64)
    err = np.abs(deq - x.astype(np.float64))
    # E4M3 keeps 4 significant bits: relative error <= 2^-4 in the normal range, and absolute
    # error <= 2^-10 * s below it
    assert (err <= np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * s[:, None]) * (1 + 1e-6)).all()
    # the largest element maps to code 448 and comes back to itself to fp32 rounding
    top = np.abs(x).argmax(axis=1)
    assert (codes[np.arange(200), top] & 0x7F == 0x7E).all()
    assert np.allclose(np.abs(deq[np.arange(200), top]), amax, rtol=2.0 ** -22, atol=0)
    z_codes, z_s = fp8.quantize_rows(np.zeros((3, 64), dtype=np.float32))
    assert (z_codes == 0).all() and (z_s == 0).all()


@pytest.mark.parametrize("D", [64, 128])
def test_k_layout_bijection_and_runs(D):
    offs = np.array([[fp8.k_byte_offset(t, d) for d in range(D)] for t in range(16)])
    assert sorted(offs.ravel().tolist()) == list(range(16 * D))
    # each (64-dim slice, token set) of 8 tokens x 64 bytes is one contiguous 512-byte run
    for p in range(D // 64):
        for sset in range(2):
            toks = [t for t in range(16) if (t // 4) % 2 == sset]
            run = offs[toks][:, 64 * p:64 * (p + 1)]
            assert run.min() == (p * 2 + sset) * 512 and run.max() == run.min() + 511


def test_fp8_cache_attention_is_attention_on_dequantised_values():
    rng = np.random.default_rng(8)
    c = Fp8CacheModel(6, 2, 64)
    k = rng.standard_normal((20, 2, 64)).astype(np.float32)
    v = rng.standard_normal((20, 2, 64)).astype(np.float32)
    slots = [3 * 16 + i for i in range(16)] + [1 * 16 + i for i in range(4)]
    c.append(k, v, slots)
    q_bits = (rng.standard_normal((1, 4, 64)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    out = oatt.paged_decode(q_bits, c, [[3, 1]], [20], 0.125, q_dtype="bf16")
    kc, ks = fp8.quantize_rows(k)
    vc, vs = fp8.quantize_rows(v)
    K = fp8.e4m3_decode(kc) * ks[..., None]
    V = fp8.e4m3_decode(vc) * vs[..., None]
    q = oatt.bits_to_f64(q_bits, "bf16")
    for h in range(4):
        ref, _ = oatt.softmax_attention(q[0, h], K[:, h // 2], V[:, h // 2], 0.125)
        assert np.allclose(out[0, h], ref, rtol=0, atol=1e-12)
    # one-token context returns the dequantised value row exactly
    one = oatt.paged_decode(q_bits, c, [[1]], [1], 0.125, q_dtype="bf16")
    assert np.array_equal(one[0, 0], V[16, 0]) and np.array_equal(one[0, 3], V[16, 1])


def _golden(name):
    with open(os.path.join(os.path.dirname(__file__), "golden", name)) as f:
        return json.load(f)


def test_fp8_k_tile_order_fixture():
    """Hand-worked byte positions of the FP8 K tile: the offset formula, and a code written by
    the model's append landing there (and nowhere else) in the stored order."""
    for case in _golden("fp8_k_tile_order.json")["cases"]:
        D, t, d, off = case["head_dim"], case["token"], case["dim"], case["byte_offset"]
        assert fp8.k_byte_offset(t, d) == off, case
        c = Fp8CacheModel(2, 2, D)
        c.k[:] = 0
        row = np.zeros((1, 2, D), dtype=np.float32)
        row[0, 1, d] = 3.0  # amax = 3 -> code 448 (0x7E) at d, code 0 elsewhere
        c.append(row, row, [16 + t])
        phys = c.k_physical()
        assert phys[1, 1, off] == 0x7E, case
        assert np.count_nonzero(phys) == 1, case


def test_fp8_v_tile_order_fixture():
    """Hand-worked byte positions of the FP8 V code tile ([dimension][16 tokens])."""
    for case in _golden("v_tile_order.json")["cases"]:
        if case["dtype"] != "fp8":
            continue
        D, t, d, off = case["head_dim"], case["token"], case["dim"], case["element_offset"]
        c = Fp8CacheModel(2, 2, D)
        c.v[:] = 0
        row = np.zeros((1, 2, D), dtype=np.float32)
        row[0, 0, d] = -0.5  # amax = 0.5 -> code -448 (0xFE) at d
        c.append(row, row, [t])
        phys = c.v_physical()
        assert phys[0, 0, off] == 0xFE, case
        assert np.count_nonzero(phys) == 1, case


def test_fp8_prefill_is_causal_attention_on_dequantised_values():
    # Chunked prefill over the quantised cache: row i at position ctx + i attends causally to the
    # values the codes stand for (code * scale), computed here from the codec alone and checked
    # with torch's fp64 causal attention, whatever blocks the table names.
    import torch
    rng = np.random.default_rng(31)
    ctx, C, Hq, Hkv, D = 19, 14, 4, 2, 64
    total = ctx + C
    c = Fp8CacheModel(5, Hkv, D)
    table = [4, 0, 2]
    k = rng.standard_normal((total, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((total, Hkv, D)).astype(np.float32)
    c.append(k, v, [table[t // 16] * 16 + t % 16 for t in range(total)])
    q_bits = (rng.standard_normal((C, Hq, D)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    out = oatt.prefill_chunk(q_bits, c, table, ctx, 0.125, q_dtype="bf16")
    kc, ks = fp8.quantize_rows(k)
    vc, vs = fp8.quantize_rows(v)
    K = fp8.e4m3_decode(kc) * ks[..., None].astype(np.float64)  # [total][Hkv][D]
    V = fp8.e4m3_decode(vc) * vs[..., None].astype(np.float64)
    q = oatt.bits_to_f64(q_bits, "bf16")
    mask = np.arange(total)[None, :] <= (ctx + np.arange(C))[:, None]
    Qt = torch.from_numpy(q.transpose(1, 0, 2))[None]
    Kt = torch.from_numpy(np.repeat(K.transpose(1, 0, 2), Hq // Hkv, axis=0))[None]
    Vt = torch.from_numpy(np.repeat(V.transpose(1, 0, 2), Hq // Hkv, axis=0))[None]
    ref = torch.nn.functional.scaled_dot_product_attention(Qt, Kt, Vt, attn_mask=torch.from_numpy(mask), scale=0.125)
    np.testing.assert_allclose(out, ref[0].numpy().transpose(1, 0, 2), rtol=0, atol=1e-12)
    # a chunk starting an empty context: its first row sees one token and returns that value row
    first = oatt.prefill_chunk(q_bits[:3], c, table, 0, 0.125, q_dtype="f16")
    assert np.array_equal(first[0, 0], V[0, 0]) and np.array_equal(first[0, 3], V[0, 1])
