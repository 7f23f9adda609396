"""GPU parity of decode over blocks shared through the prefix cache ([Serving] The Build, Step 8).

A request whose prompt starts with a registered prefix gets those blocks from
pkv_prefix_lookup, appends only its own tokens, and its decode must equal the oracle's and, bit
for bit, the decode of the same tokens laid out in private blocks.  After the shared blocks are
released and evicted by a large allocation, a new request must match less and still decode
correctly from the recycled blocks."""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import attention as oatt
from paged_kv_cache_404_amd import ops

from .gpu_util import ATOL, Mirror, i32, to_dev

pytestmark = pytest.mark.gpu

HQ, HKV, D = 32, 8, 128


def _decode(m, seqs, q_bits, ps=0):
    tables, lens = m.tables(seqs)
    mcl = int(lens.max())
    out = torch.full((len(seqs), HQ, D), float("nan"), dtype=torch.float32, device="cuda")
    ops.paged_attention_decode(out, to_dev(q_bits, "bf16"), m.k, m.v, i32(tables), i32(lens), mcl, 1 / np.sqrt(D), ps,
                               ops.decode_workspace(len(seqs), HQ, D, mcl, ps))
    torch.cuda.synchronize()
    ref = oatt.paged_decode(q_bits, m.cache, tables, lens, 1 / np.sqrt(D))
    assert float(np.abs(out.cpu().numpy().astype(np.float64) - ref).max()) <= ATOL
    return out


@pytest.mark.parametrize("ps", [0, 512])
def test_prefix_hit_decodes_like_private_blocks(ps):
    rng = np.random.default_rng(61 + ps)
    N = 420
    m = Mirror(N, HKV, D, "bf16", rng.permutation(N))
    prompt = [int(x) for x in rng.integers(0, 32000, 2040)]
    a = m.new_seq()
    ka, va = wl.normal_bits(rng, (2040, HKV, D), "bf16"), wl.normal_bits(rng, (2040, HKV, D), "bf16")
    m.append([a], [2040], ka, va)
    assert m.prefix_insert(a, prompt) == 127  # the full blocks of 2,040 tokens
    # request b: the same 2,040-token prompt and 30 tokens of its own
    tb = prompt + [int(x) for x in rng.integers(0, 32000, 30)]
    b, n = m.prefix_lookup(tb)
    assert n == 2032
    kb, vb = wl.normal_bits(rng, (38, HKV, D), "bf16"), wl.normal_bits(rng, (38, HKV, D), "bf16")
    kb[:8], vb[:8] = ka[2032:], va[2032:]  # positions 2032..2039 carry the prompt's K/V again
    m.append([b], [38], kb, vb)
    m.assert_cache_bit_exact()
    # the same sequence content in private blocks
    c = m.new_seq()
    m.append([c], [2070], np.concatenate([ka, kb[8:]]), np.concatenate([va, vb[8:]]))
    q = wl.normal_bits(rng, (1, HQ, D), "bf16")
    ob = _decode(m, [b], q, ps)
    oc = _decode(m, [c], q, ps)
    assert torch.equal(ob.view(torch.int32), oc.view(torch.int32))
    # release everything: the registered blocks wait on the LRU
    for s in (a, b, c):
        m.free(s)
    assert len(m.opool.lru) == 127
    # a 6,000-token sequence needs 375 blocks: the free list has 293, so the 82 deepest registered
    # blocks are evicted and the first 45 blocks (720 tokens) of the prompt stay registered
    big = m.new_seq()
    m.append([big], [6000], wl.normal_bits(rng, (6000, HKV, D), "bf16"), wl.normal_bits(rng, (6000, HKV, D), "bf16"))
    assert m.pool.num_free() == 0 and len(m.opool.entries) == 45
    d, n2 = m.prefix_lookup(tb)
    assert n2 == 720
    m.free(big)  # d's own tokens land in blocks that held the evicted prompt blocks and big's data
    rest = len(tb) - n2
    kd, vd = wl.normal_bits(rng, (rest, HKV, D), "bf16"), wl.normal_bits(rng, (rest, HKV, D), "bf16")
    kd[: 2040 - 720], vd[: 2040 - 720] = ka[720:], va[720:]
    m.append([d], [rest], kd, vd)
    m.assert_cache_bit_exact()
    od = _decode(m, [d], q, ps)
    e = m.new_seq()  # the same content again, in private blocks
    m.append([e], [2070], np.concatenate([ka, kd[2040 - 720:]]), np.concatenate([va, vd[2040 - 720:]]))
    oe = _decode(m, [e], q, ps)
    assert torch.equal(od.view(torch.int32), oe.view(torch.int32))
