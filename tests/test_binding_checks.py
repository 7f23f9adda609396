"""The Python binding rejects mismatched tensors before any launch (CPU tensors; nothing here
reaches a GPU).  Shapes and dtypes are checked before the tensors' device, so each case below
fails on its own mismatch."""
import pytest
import torch

from paged_kv_cache_404_amd import ops

N, HKV, HQ, D = 8, 2, 8, 64


def _cache(dtype=torch.bfloat16, tile=16 * D):
    return torch.empty((N, HKV, tile), dtype=dtype), torch.empty((N, HKV, tile), dtype=dtype)


def test_cache_tensors_are_flat_tiles():
    k, v = _cache()
    assert ops.cache_dims(k, v) == (N, HKV, D)
    assert ops.cache_dims(k, v, D) == (N, HKV, D)
    with pytest.raises(ValueError, match="head_dim"):
        ops.cache_dims(k, v, 128)
    # the [16][D] / [D][16] shapes that index as if they named (token, dimension) are refused
    with pytest.raises(ValueError, match="tiles"):
        ops.cache_dims(torch.empty((N, HKV, 16, D)), torch.empty((N, HKV, D, 16)))
    with pytest.raises(ValueError, match="tiles"):
        ops.cache_dims(k, torch.empty((N, HKV + 1, 16 * D)))
    with pytest.raises(ValueError, match="tiles"):
        ops.cache_dims(torch.empty((N, HKV, 100)), torch.empty((N, HKV, 100)))


def _mixed(**kw):
    k, v = _cache()
    B, C = 3, 20
    a = dict(dec_out=torch.empty((B, HQ, D)), dec_query=torch.empty((B, HQ, D), dtype=torch.bfloat16),
             dec_tables=torch.zeros((B, 4), dtype=torch.int32), dec_lens=torch.ones(B, dtype=torch.int32),
             dec_max_context_len=64, pre_out=torch.empty((C, HQ, D)),
             pre_query=torch.empty((C, HQ, D), dtype=torch.bfloat16), pre_tables=torch.zeros((1, 4), dtype=torch.int32),
             ctx_starts=[10], chunk_lens=[C], k_cache=k, v_cache=v, scale=0.125, host_dec_lens=None)
    a.update(kw)
    return ops._mixed_args(**a)


@pytest.mark.parametrize("change,err,match", [
    (dict(dec_out=torch.empty((3, HQ, D), dtype=torch.bfloat16)), TypeError, "share one dtype"),
    (dict(pre_out=torch.empty((20, HQ, D), dtype=torch.bfloat16)), TypeError, "share one dtype"),
    (dict(dec_out=torch.empty((3, HQ, 2 * D))), ValueError, "dec_out"),
    (dict(dec_query=torch.empty((3, HQ, 2 * D), dtype=torch.bfloat16),
          dec_out=torch.empty((3, HQ, 2 * D))), ValueError, "dec_query"),
    (dict(dec_query=torch.empty((3, 2 * HQ, D), dtype=torch.bfloat16),
          dec_out=torch.empty((3, 2 * HQ, D))), ValueError, "same number of heads"),
    (dict(dec_query=torch.empty((3, HQ, D), dtype=torch.float16)), TypeError, "dec_query"),
    (dict(pre_query=torch.empty((20, HQ, D), dtype=torch.float16)), TypeError, "pre_query"),
    (dict(dec_lens=torch.ones((3, 1), dtype=torch.int32)), ValueError, "lens"),
    (dict(dec_tables=torch.zeros(12, dtype=torch.int32)), ValueError, "tables"),
    (dict(dec_tables=torch.zeros((4, 4), dtype=torch.int32)), ValueError, "tables"),
    (dict(dec_lens=torch.ones(3, dtype=torch.int64)), TypeError, "int32"),
    (dict(chunk_lens=[19]), ValueError, "sum"),
    (dict(ctx_starts=[10, 0]), ValueError, "one entry per chunk"),
    (dict(pre_tables=torch.zeros((2, 4), dtype=torch.int32)), ValueError, "prefill tables"),
])
def test_mixed_mismatches_raise_before_launch(change, err, match):
    with pytest.raises(err, match=match):
        _mixed(**change)


def test_mixed_valid_cpu_arguments_stop_at_the_device_check():
    with pytest.raises(ValueError, match="GPU"):
        _mixed()
