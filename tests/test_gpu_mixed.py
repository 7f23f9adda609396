"""GPU parity of the mixed decode + prefill launch (paged_attention_mixed).

Its outputs must equal, bit for bit, those of the separate launches it replaces
(paged_attention_decode with the same partition size, and paged_attention_prefill_chunk per chunk),
and lie within 2e-3 of the oracle.  Cases cover several chunks (including a first chunk at position 0
and ragged lengths), either part empty, the longest-first order, every group size (1, 2, 4, 8
query heads per KV head), head dims 64 and 128, fp16, a 16-bit output, split-K partitions in the
decode part (merged by the reduce launch that follows), decode sequences grouped to share their
common blocks, and the prefix-sharing step of 16 samples plus a 512-row chunk over a 4,096-token
context, plain and grouped, single pass and split-K."""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import attention as oatt
from paged_kv_cache_404_amd import PKV_EUNSUPPORTED, PagedKVError, ops

from .gpu_util import ATOL, Mirror, i32, to_dev

pytestmark = pytest.mark.gpu


def _scene(seed, dec_lens, chunks, Hq, Hkv, D, dtype):
    """Decode sequences with dec_lens tokens cached; prefill sequences with ctx + C cached."""
    rng = np.random.default_rng(seed)
    need = sum(-(-L // 16) for L in dec_lens) + sum(-(-(c + n) // 16) for c, n in chunks)
    N = need + 8
    m = Mirror(N, Hkv, D, dtype, rng.permutation(N))
    dseqs = [m.new_seq() for _ in dec_lens]
    pseqs = [m.new_seq() for _ in chunks]
    counts = list(dec_lens) + [c + n for c, n in chunks]
    tot = sum(counts)
    if tot:
        m.append(dseqs + pseqs, counts, wl.normal_bits(rng, (tot, Hkv, D), dtype),
                 wl.normal_bits(rng, (tot, Hkv, D), dtype))
    q_dec = wl.normal_bits(rng, (len(dec_lens), Hq, D), dtype)
    q_pre = wl.normal_bits(rng, (sum(n for _, n in chunks), Hq, D), dtype)
    return m, dseqs, pseqs, q_dec, q_pre


def _run(m, dseqs, pseqs, chunks, q_dec, q_pre, Hq, D, dtype, scale, out_dtype=torch.float32, host_lens=False,
         ps=0, ns=1):
    B, S = len(dseqs), len(pseqs)
    dtab, dlens = m.tables(dseqs) if B else (None, None)
    ptab, _ = m.tables(pseqs) if S else (None, None)
    R = int(q_pre.shape[0])
    mcl = int(dlens.max()) if B else 0
    ws = ops.decode_workspace(B, Hq, D, mcl, ps) if (B and ps > 0) else None
    dec_sep = torch.full((B, Hq, D), float("nan"), dtype=out_dtype, device="cuda")
    pre_sep = torch.full((R, Hq, D), float("nan"), dtype=out_dtype, device="cuda")
    if B:
        ops.paged_attention_decode(dec_sep, to_dev(q_dec, dtype), m.k, m.v, i32(dtab), i32(dlens), mcl, scale, ps, ws)
    r0 = 0
    for i, (c, n) in enumerate(chunks):
        if n:
            ops.paged_attention_prefill_chunk(pre_sep[r0:r0 + n], to_dev(q_pre[r0:r0 + n], dtype), m.k, m.v,
                                              i32(ptab[i]), c, scale)
        r0 += n
    dec_mix = torch.full_like(dec_sep, float("nan"))
    pre_mix = torch.full_like(pre_sep, float("nan"))
    ws2 = torch.full_like(ws, 0xFF) if ws is not None else None  # NaN partials until written
    ops.paged_attention_mixed(dec_mix if B else None, to_dev(q_dec, dtype) if B else None,
                              i32(dtab) if B else None, i32(dlens) if B else None,
                              mcl, pre_mix if S else None,
                              to_dev(q_pre, dtype) if S else None, i32(ptab) if S else None,
                              [c for c, _ in chunks], [n for _, n in chunks], m.k, m.v, scale,
                              host_dec_lens=dlens if (B and host_lens) else None, dec_partition_size=ps,
                              dec_group_size=ns, workspace=ws2)
    torch.cuda.synchronize()
    view = torch.int32 if out_dtype == torch.float32 else torch.int16
    assert torch.equal(dec_mix.view(view), dec_sep.view(view))
    assert torch.equal(pre_mix.view(view), pre_sep.view(view))
    return dec_mix, pre_mix, dtab, dlens, ptab


def _check_oracle(m, dec, pre, dtab, dlens, ptab, q_dec, q_pre, chunks, scale):
    if dtab is not None:
        ref = oatt.paged_decode(q_dec, m.cache, dtab, dlens, scale)
        assert float(np.abs(dec.float().cpu().numpy().astype(np.float64) - ref).max()) <= ATOL
    r0 = 0
    for i, (c, n) in enumerate(chunks):
        ref = oatt.prefill_chunk(q_pre[r0:r0 + n], m.cache, ptab[i], c, scale)
        assert float(np.abs(pre[r0:r0 + n].float().cpu().numpy().astype(np.float64) - ref).max()) <= ATOL
        r0 += n


CASES = [
    # seed, decode lengths, chunks (ctx_start, length), Hq, Hkv, D, dtype
    (1, [1, 17, 300, 2048, 513, 64], [(0, 37), (100, 16), (640, 130)], 32, 8, 128, "bf16"),
    (2, [5, 900], [(33, 1)], 32, 8, 128, "bf16"),
    (3, [], [(0, 20), (48, 64)], 32, 8, 128, "bf16"),
    (4, [1000, 2, 700], [], 32, 8, 128, "bf16"),
    (5, [40, 129, 1500], [(16, 48), (0, 5)], 64, 8, 64, "f16"),
    (6, [77, 31], [(250, 130)], 16, 4, 64, "bf16"),
    (7, [30, 600, 1, 250], [(0, 16), (300, 70)], 16, 8, 128, "bf16"),   # 2 query heads per KV head
    (8, [130, 7, 1025], [(17, 40), (0, 33)], 8, 8, 128, "bf16"),        # 1 query head per KV head
    (9, [64, 700], [(90, 100)], 8, 4, 64, "f16"),
]


@pytest.mark.parametrize("seed,dec_lens,chunks,Hq,Hkv,D,dtype", CASES)
def test_mixed_equals_separate_launches(seed, dec_lens, chunks, Hq, Hkv, D, dtype):
    m, dseqs, pseqs, q_dec, q_pre = _scene(seed, dec_lens, chunks, Hq, Hkv, D, dtype)
    scale = 1 / np.sqrt(D)
    dec, pre, dtab, dlens, ptab = _run(m, dseqs, pseqs, chunks, q_dec, q_pre, Hq, D, dtype, scale,
                                       host_lens=seed % 2 == 1)
    _check_oracle(m, dec, pre, dtab, dlens, ptab, q_dec, q_pre, chunks, scale)


@pytest.mark.parametrize("seed,ps,ns", [(1, 512, 1), (1, 64, 1), (7, 256, 1), (8, 1024, 1), (1, 0, 2), (1, 512, 2),
                                        (7, 0, 4), (8, 128, 8), (5, 64, 2), (9, 256, 4)])
def test_mixed_split_k_and_grouped_decode(seed, ps, ns):
    """The decode part with split-K partitions (4-wave partitions up to 512 tokens, 8 above) and
    grouped sequences: bit for bit paged_attention_decode with the same partition size."""
    case = [c for c in CASES if c[0] == seed][0]
    _, dec_lens, chunks, Hq, Hkv, D, dtype = case
    m, dseqs, pseqs, q_dec, q_pre = _scene(seed, dec_lens, chunks, Hq, Hkv, D, dtype)
    scale = 1 / np.sqrt(D)
    dec, pre, dtab, dlens, ptab = _run(m, dseqs, pseqs, chunks, q_dec, q_pre, Hq, D, dtype, scale,
                                       host_lens=True, ps=ps, ns=ns)
    _check_oracle(m, dec, pre, dtab, dlens, ptab, q_dec, q_pre, chunks, scale)


F32_CASES = [
    # seed, decode lengths, chunks, Hq, Hkv, D, partition size
    (11, [5, 17, 32, 40], [(0, 8), (24, 9)], 8, 8, 64, 0),          # the tiny step's shape
    (12, [1, 300, 64, 1000], [(0, 37), (100, 16), (640, 130)], 16, 4, 128, 0),
    (13, [129, 700, 2], [(33, 70)], 32, 8, 64, 256),
    (14, [], [(0, 20), (48, 64)], 8, 2, 128, 0),
    (15, [900, 3], [], 16, 8, 64, 64),
]


@pytest.mark.parametrize("seed,dec_lens,chunks,Hq,Hkv,D,ps", F32_CASES)
def test_mixed_fp32_equals_separate_launches(seed, dec_lens, chunks, Hq, Hkv, D, ps):
    """fp32 caches: the mixed launch runs the vector-ALU decode and prefill bodies, bit for bit the
    fp32 decode (split-K included) and fp32 prefill launches, and within 2e-3 of the oracle."""
    m, dseqs, pseqs, q_dec, q_pre = _scene(seed, dec_lens, chunks, Hq, Hkv, D, "f32")
    scale = 1 / np.sqrt(D)
    dec, pre, dtab, dlens, ptab = _run(m, dseqs, pseqs, chunks, q_dec, q_pre, Hq, D, "f32", scale,
                                       host_lens=seed % 2 == 1, ps=ps)
    _check_oracle(m, dec, pre, dtab, dlens, ptab, q_dec, q_pre, chunks, scale)


def test_mixed_fp32_rejects_grouping():
    chunks = [(0, 16)]
    m, dseqs, pseqs, q_dec, q_pre = _scene(16, [40, 50], chunks, 8, 8, 64, "f32")
    with pytest.raises(PagedKVError) as e:
        _run(m, dseqs, pseqs, chunks, q_dec, q_pre, 8, 64, "f32", 0.125, ns=8)
    assert e.value.status == PKV_EUNSUPPORTED


def test_mixed_output_in_bf16():
    chunks = [(64, 64)]
    m, dseqs, pseqs, q_dec, q_pre = _scene(9, [300, 45], chunks, 32, 8, 128, "bf16")
    _run(m, dseqs, pseqs, chunks, q_dec, q_pre, 32, 128, "bf16", 0.088, out_dtype=torch.bfloat16)
    _run(m, dseqs, pseqs, chunks, q_dec, q_pre, 32, 128, "bf16", 0.088, out_dtype=torch.bfloat16, ps=128, ns=2)


def _prefix_step(prefix_len):
    mw = wl.mixed_step(5, prefix_len=prefix_len)
    rng = mw.rng
    m = Mirror(mw.num_blocks, mw.Hkv, mw.D, mw.dtype, mw.free_order)
    s0 = m.new_seq()
    m.append([s0], [mw.prefix_len], wl.normal_bits(rng, (mw.prefix_len, mw.Hkv, mw.D), mw.dtype),
             wl.normal_bits(rng, (mw.prefix_len, mw.Hkv, mw.D), mw.dtype))
    samples = [s0] + [m.fork(s0) for _ in range(mw.samples - 1)]
    pf = m.new_seq()
    m.append([pf], [mw.ctx_start], wl.normal_bits(rng, (mw.ctx_start, mw.Hkv, mw.D), mw.dtype),
             wl.normal_bits(rng, (mw.ctx_start, mw.Hkv, mw.D), mw.dtype))
    _, cow = m.append(samples + [pf], [1] * mw.samples + [mw.chunk],
                      wl.normal_bits(rng, (mw.samples + mw.chunk, mw.Hkv, mw.D), mw.dtype),
                      wl.normal_bits(rng, (mw.samples + mw.chunk, mw.Hkv, mw.D), mw.dtype))
    assert len(cow) == (0 if prefix_len % 16 == 0 else mw.samples - 1)
    q_dec = wl.normal_bits(rng, (mw.samples, mw.Hq, mw.D), mw.dtype)
    q_pre = wl.normal_bits(rng, (mw.chunk, mw.Hq, mw.D), mw.dtype)
    return mw, m, samples, pf, q_dec, q_pre


@pytest.mark.parametrize("prefix_len,ps,ns", [(2048, 0, 1), (2048, 0, 2), (2048, 512, 2), (2040, 512, 2), (2040, 0, 1)])
def test_mixed_prefix_sharing_step(prefix_len, ps, ns):
    """16 samples forked from a 2,048-token prefix (or a 2,040-token one, whose partial last block
    was copied on write for 15 of them) decode one token each, and a 512-row chunk is prefilled
    after 4,096 cached tokens, in one launch: every decode output and every chunk row against the
    oracle, bit for bit against the separate launches."""
    mw, m, samples, pf, q_dec, q_pre = _prefix_step(prefix_len)
    chunks = [(mw.ctx_start, mw.chunk)]
    dec, pre, dtab, dlens, ptab = _run(m, samples, [pf], chunks, q_dec, q_pre, mw.Hq, mw.D, mw.dtype, mw.scale,
                                       host_lens=True, ps=ps, ns=ns)
    _check_oracle(m, dec, pre, dtab, dlens, ptab, q_dec, q_pre, chunks, mw.scale)


@pytest.mark.parametrize("ns", [3, 4, 8])
def test_mixed_rejects_other_group_sizes(ns):
    m, dseqs, pseqs, q_dec, q_pre = _scene(8, [30], [(0, 16)], 32, 8, 128, "bf16")
    dtab, dlens = m.tables(dseqs)
    ptab, _ = m.tables(pseqs)
    out = torch.empty((1, 32, 128), device="cuda")
    pout = torch.empty((16, 32, 128), device="cuda")
    with pytest.raises(PagedKVError) as e:
        ops.paged_attention_mixed(out, to_dev(q_dec, "bf16"), i32(dtab), i32(dlens), 30, pout, to_dev(q_pre, "bf16"),
                                  i32(ptab), [0], [16], m.k, m.v, 0.1, dec_group_size=ns)
    assert e.value.status == PKV_EUNSUPPORTED
