"""Continuous-batching trace (512 Poisson-arriving requests, lognormal prompts, geometric outputs,
at most 128 running, 32q/8kv x 128 bf16): the library's pool and the oracle's pool agree on every
slot, table, length, free list and out-of-blocks decision over the whole trace; on the GPU, every
step's append + split-K decode runs through the C ABI and sampled steps match the fp64 oracle."""
import pytest

from .trace_driver import run_trace


@pytest.mark.parametrize("num_blocks,preempts", [(12288, False), (3072, True)])
def test_trace_pool_parity(num_blocks, preempts):
    st = run_trace(num_blocks=num_blocks, gpu=False)
    assert st.finished == 512 and st.seq_steps > 100_000
    assert st.max_active == (128 if not preempts else st.max_active)
    assert (st.preemptions > 0) == preempts
    assert st.admissions == 512 + st.preemptions
    # [Chapter] "PagedAttention: KV cache memory": with 16-token blocks under 4 % of the
    # allocated cache is wasted; here the tail of each sequence's last block is all that is.
    assert st.min_utilisation > 0.96


@pytest.mark.gpu
def test_trace_gpu_full():
    st = run_trace(num_blocks=12288, gpu=True, check_every=100)
    assert not st.errors, st.errors
    assert st.attention_checks >= 17 and st.max_abs_err <= 2e-3
    print(f"trace: {st.steps} steps, {st.seq_steps} seq-steps, max |err| {st.max_abs_err:.2e}")


@pytest.mark.gpu
def test_trace_gpu_preemption():
    # 64 requests through a 2,048-block pool: preemption and recompute happen (10 times)
    st = run_trace(num_blocks=2048, n_requests=64, gpu=True, check_every=50)
    assert st.preemptions > 0
    assert not st.errors, st.errors
    assert st.attention_checks >= 15 and st.max_abs_err <= 2e-3
