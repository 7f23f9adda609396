"""torch-tensor wrappers over the device calls of libpagedkv (argument marshalling only).

Every computation happens in the HIP kernels; these functions check dtype, device and
contiguity, then pass raw pointers and the current HIP stream to the C ABI.
"""
from __future__ import annotations

import numpy as np
import torch

from ._lib import PKV_BF16, PKV_F16, PKV_F32, check, lib

_DT = {torch.float32: PKV_F32, torch.float16: PKV_F16, torch.bfloat16: PKV_BF16}


def dtype_code(t: torch.dtype) -> int:
    if t not in _DT:
        raise TypeError(f"unsupported dtype {t}")
    return _DT[t]


def _dev(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _stream(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


# ---- cache tensors ---------------------------------------------------------------------------
# One layer's K and V caches are two tensors of shape [num_blocks][num_kv_heads][16 * head_dim]:
# entry [b, h, :] is the whole (block, head) tile, in the stored order include/pagedkv.h defines
# (the K tile as 16-byte operand chunks, the V tile as [token half][head_dim][8 tokens]).  The last
# axis is deliberately flat: a [16][head_dim] shape would invite k[b, h, t, d] indexing, which does
# not name token t's dimension d.  Write the cache with paged_cache_append only.

def kv_cache(num_blocks: int, num_kv_heads: int, head_dim: int, dtype=torch.bfloat16, device="cuda"):
    """Allocate an uninitialised (k_cache, v_cache) pair, each [num_blocks][num_kv_heads][16 * head_dim]."""
    shape = (num_blocks, num_kv_heads, 16 * head_dim)
    return torch.empty(shape, dtype=dtype, device=device), torch.empty(shape, dtype=dtype, device=device)


def cache_dims(k_cache, v_cache, head_dim: int | None = None):
    """(num_blocks, num_kv_heads, head_dim) of a cache pair; checks the flat tile shape."""
    if k_cache.dim() != 3 or tuple(v_cache.shape) != tuple(k_cache.shape) or k_cache.shape[2] % 16:
        raise ValueError("k_cache and v_cache must both be [num_blocks][num_kv_heads][16 * head_dim] tiles")
    N, H, tile = k_cache.shape
    D = tile // 16
    if head_dim is not None and head_dim != D:
        raise ValueError(f"cache tiles hold head_dim {D}, the call has {head_dim}")
    return N, H, D


def paged_cache_append(k_cache, v_cache, key, value, slot_mapping, stream=None) -> None:
    """k_cache/v_cache [N][Hkv][16 * D] tiles (kv_cache); key/value [T][Hkv][D]; slot_mapping int32 [T]."""
    _dev(k_cache, v_cache, key, value, slot_mapping)
    N, H, D = cache_dims(k_cache, v_cache, key.shape[-1] if key.dim() == 3 else None)
    bs = 16
    if key.dtype != k_cache.dtype or value.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype:
        raise TypeError("key, value and caches must share one dtype")
    if slot_mapping.dtype != torch.int32:
        raise TypeError("slot_mapping must be int32")
    T = slot_mapping.numel()
    if key.shape != (T, H, D) or value.shape != (T, H, D):
        raise ValueError("key/value must be [T][Hkv][D]")
    check(lib.paged_cache_append(k_cache.data_ptr(), v_cache.data_ptr(), key.data_ptr(), value.data_ptr(), 0, 0,
                                 slot_mapping.data_ptr(), T, H, D, bs, N, dtype_code(k_cache.dtype), _stream(stream)))


def paged_cache_copy_blocks(k_cache, v_cache, src_dst, stream=None) -> None:
    """src_dst int32 [n][2] on the GPU."""
    _dev(k_cache, v_cache, src_dst)
    N, H, D = cache_dims(k_cache, v_cache)
    bs = 16
    if src_dst.dtype != torch.int32 or src_dst.dim() != 2 or src_dst.shape[1] != 2:
        raise ValueError("src_dst must be int32 [n][2]")
    check(lib.paged_cache_copy_blocks(k_cache.data_ptr(), v_cache.data_ptr(), src_dst.data_ptr(), src_dst.shape[0],
                                      H, D, bs, N, dtype_code(k_cache.dtype), _stream(stream)))


def check_inputs(num_blocks: int, block_tables=None, context_lens=None, max_context_len: int = 0,
                 slot_mapping=None, block_size: int = 16, stream=None) -> dict:
    """paged_check_inputs: counts the block-table, length and slot values the kernels would clamp
    or skip.  This helper waits for the result (the C call itself does not synchronise)."""
    B = 0 if context_lens is None else context_lens.numel()
    T = 0 if slot_mapping is None else slot_mapping.numel()
    tensors = [t for t in (block_tables, context_lens, slot_mapping) if t is not None]
    if tensors:
        _dev(*tensors)
    for t in tensors:
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError("block_tables, context_lens and slot_mapping must be contiguous int32")
    if B and (block_tables is None or block_tables.dim() != 2 or block_tables.shape[0] != B):
        raise ValueError("block_tables must be [B][max_blocks_per_seq]")
    dev = tensors[0].device if tensors else torch.device("cuda")
    counts = torch.empty(4, dtype=torch.int32, device=dev)
    check(lib.paged_check_inputs(block_tables.data_ptr() if B else None, context_lens.data_ptr() if B else None, B,
                                 block_tables.shape[1] if B else 0, int(max_context_len),
                                 slot_mapping.data_ptr() if T else None, T, int(num_blocks), int(block_size),
                                 counts.data_ptr(), _stream(stream)))
    c = counts.cpu().tolist()
    return {"bad_lengths": c[0], "bad_block_ids": c[1], "first_bad_sequence": None if c[2] == 2147483647 else c[2],
            "bad_slots": c[3]}


def probe_stream_read(buf, nbytes: int, sink, workgroups: int = 2048, stream=None) -> None:
    """paged_probe_stream_read over the first nbytes of buf (a measuring aid, no result)."""
    _dev(buf, sink)
    if nbytes > buf.numel() * buf.element_size():
        raise ValueError("nbytes exceeds the buffer")
    check(lib.paged_probe_stream_read(buf.data_ptr(), int(nbytes), sink.data_ptr(), int(workgroups), _stream(stream)))


def decode_workspace_bytes(B: int, Hq: int, D: int, max_context_len: int, partition_size: int) -> int:
    return int(lib.paged_attention_decode_workspace_bytes(B, Hq, D, max_context_len, partition_size))


def decode_workspace(B: int, Hq: int, D: int, max_context_len: int, partition_size: int, device="cuda"):
    n = decode_workspace_bytes(B, Hq, D, max_context_len, partition_size)
    return torch.empty(max(n, 16), dtype=torch.uint8, device=device)


def _host_lens_ptr(host_context_lens):
    if host_context_lens is None:
        return None, None
    hl = np.ascontiguousarray(np.asarray(host_context_lens, dtype=np.int32))
    return hl, hl.ctypes.data


def _decode_args(out, query, k_cache, v_cache, block_tables, context_lens, max_context_len, scale, partition_size,
                 workspace, host_ptr=None):
    _dev(out, query, k_cache, v_cache, block_tables, context_lens)
    if query.dim() != 3:
        raise ValueError("query must be [B][Hq][D]")
    B, Hq, D = query.shape
    N, Hkv, _ = cache_dims(k_cache, v_cache, D)
    bs = 16
    if out.shape != query.shape:
        raise ValueError("out must be [B][Hq][D]")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [B][max_blocks], context_lens [B]")
    if query.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype:
        raise TypeError("query and caches must share one dtype")
    ws_ptr, ws_bytes = (0, 0) if workspace is None else (workspace.data_ptr(), workspace.numel() * workspace.element_size())
    return (out.data_ptr(), dtype_code(out.dtype), query.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            block_tables.data_ptr(), context_lens.data_ptr(), B, Hq, Hkv, D, bs, block_tables.shape[1], N,
            int(max_context_len), float(scale), int(partition_size), ws_ptr, ws_bytes, dtype_code(k_cache.dtype),
            host_ptr)


def paged_attention_decode(out, query, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                           partition_size=0, workspace=None, stream=None, host_context_lens=None) -> None:
    """host_context_lens: optional host copy of context_lens, used only to order the work."""
    hl, hp = _host_lens_ptr(host_context_lens)
    args = _decode_args(out, query, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                        partition_size, workspace, hp)
    check(lib.paged_attention_decode(*args, _stream(stream)))


def paged_attention_decode_grouped(out, query, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                                   group_size, partition_size=0, workspace=None, stream=None) -> None:
    """Decode in which batch rows group_size*k .. group_size*k + group_size - 1 share a workgroup and
    read the blocks common to their tables once; output bit for bit paged_attention_decode's."""
    args = _decode_args(out, query, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                        partition_size, workspace)
    check(lib.paged_attention_decode_grouped(*args[:20], int(group_size), _stream(stream)))


def paged_attention_decode_noalloc(out, query, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                                   partition_size=0, stream=None, host_context_lens=None) -> None:
    """paged_attention_decode with the split-K partials in the library's static per-GPU scratch
    (no workspace argument, nothing allocated).  Calls that overlap on one GPU race."""
    hl, hp = _host_lens_ptr(host_context_lens)
    args = _decode_args(out, query, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                        partition_size, None, hp)
    check(lib.paged_attention_decode_noalloc(*args[:17], args[19], args[20], _stream(stream)))


def _fused_args(args, new_key, new_value):
    """Argument tuple of the fused-append entry points from a _decode_args tuple."""
    _dev(new_key, new_value)
    B, Hkv, D = args[7], args[9], args[10]
    for t in (new_key, new_value):
        if tuple(t.shape) != (B, Hkv, D) or dtype_code(t.dtype) != args[19]:
            raise ValueError("new_key/new_value must be [B][Hkv][D] of the cache dtype")
    return args[:3] + (new_key.data_ptr(), new_value.data_ptr()) + args[3:]


def paged_attention_decode_append(out, query, new_key, new_value, k_cache, v_cache, block_tables, context_lens,
                                  max_context_len, scale, partition_size=0, workspace=None, stream=None,
                                  host_context_lens=None) -> None:
    """One decode step with the append fused in: token context_lens[b] - 1 of every sequence
    (new_key/new_value [B][Hkv][D]) is written to its slot and attended over."""
    hl, hp = _host_lens_ptr(host_context_lens)
    args = _decode_args(out, query, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                        partition_size, workspace, hp)
    check(lib.paged_attention_decode_append(*_fused_args(args, new_key, new_value), _stream(stream)))


def paged_attention_decode_newest(out, query, new_key, new_value, k_cache, v_cache, block_tables, context_lens,
                                  max_context_len, scale, partition_size=0, workspace=None, stream=None,
                                  host_context_lens=None) -> None:
    """Decode with every sequence's newest token (position context_lens[b] - 1) taken from
    new_key/new_value; the cache is not written (append those tokens with paged_cache_append,
    possibly concurrently on another stream)."""
    hl, hp = _host_lens_ptr(host_context_lens)
    args = _decode_args(out, query, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                        partition_size, workspace, hp)
    check(lib.paged_attention_decode_newest(*_fused_args(args, new_key, new_value), _stream(stream)))


def paged_attention_decode_append_partitions(out, query, new_key, new_value, k_cache, v_cache, block_tables,
                                             context_lens, max_context_len, scale, partition_size, workspace,
                                             stream=None) -> None:
    """paged_attention_decode_append's split-K as two launches: this, then paged_attention_decode_reduce."""
    args = _decode_args(out, query, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                        partition_size, workspace)
    check(lib.paged_attention_decode_append_partitions(*_fused_args(args, new_key, new_value), _stream(stream)))


def paged_attention_decode_newest_partitions(out, query, new_key, new_value, k_cache, v_cache, block_tables,
                                             context_lens, max_context_len, scale, partition_size, workspace,
                                             stream=None) -> None:
    """paged_attention_decode_newest's split-K as two launches: this, then paged_attention_decode_reduce."""
    args = _decode_args(out, query, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                        partition_size, workspace)
    check(lib.paged_attention_decode_newest_partitions(*_fused_args(args, new_key, new_value), _stream(stream)))


def paged_attention_decode_partitions(out, query, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                                      partition_size, workspace, stream=None) -> None:
    args = _decode_args(out, query, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                        partition_size, workspace)
    check(lib.paged_attention_decode_partitions(*args, _stream(stream)))


def paged_attention_decode_reduce(out, context_lens, max_context_len, partition_size, workspace, stream=None) -> None:
    _dev(out, context_lens, workspace)
    B, Hq, D = out.shape
    check(lib.paged_attention_decode_reduce(out.data_ptr(), dtype_code(out.dtype), context_lens.data_ptr(), B, Hq, D,
                                            int(max_context_len), int(partition_size), workspace.data_ptr(),
                                            workspace.numel() * workspace.element_size(), _stream(stream)))


def _prefill_args(out, query, k_cache, v_cache, block_table, ctx_start, scale):
    _dev(out, query, k_cache, v_cache, block_table)
    if query.dim() != 3 or out.shape != query.shape:
        raise ValueError("query and out must be [C][Hq][D]")
    C, Hq, D = query.shape
    N, Hkv, _ = cache_dims(k_cache, v_cache, D)
    bs = 16
    if query.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype:
        raise TypeError("query and caches must share one dtype")
    if block_table.dtype != torch.int32:
        raise TypeError("block_table must be int32")
    if block_table.numel() * bs < ctx_start + C:
        raise ValueError("block_table too short for ctx_start + C")
    return (out.data_ptr(), dtype_code(out.dtype), query.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            block_table.data_ptr(), int(ctx_start), C, Hq, Hkv, D, bs, N, float(scale), dtype_code(k_cache.dtype))


class PreparedPrefill:
    """paged_attention_prefill_chunk with its arguments marshalled once."""

    def __init__(self, out, query, k_cache, v_cache, block_table, ctx_start, scale, stream=None):
        self._keep = (out, query, k_cache, v_cache, block_table)
        self.args = _prefill_args(out, query, k_cache, v_cache, block_table, ctx_start, scale)
        self.stream = _stream(stream)

    def __call__(self) -> None:
        check(lib.paged_attention_prefill_chunk(*self.args, self.stream))


def paged_attention_prefill_chunk(out, query, k_cache, v_cache, block_table, ctx_start, scale, stream=None) -> None:
    """query/out [C][Hq][D]; block_table int32 [>= ceil((ctx_start + C) / 16)] of one sequence."""
    check(lib.paged_attention_prefill_chunk(*_prefill_args(out, query, k_cache, v_cache, block_table, ctx_start,
                                                           scale), _stream(stream)))


class PreparedDecode:
    """Decode call with its arguments marshalled once, for tight step loops: each call is one
    C-ABI call (the tensors must stay alive and unchanged in shape)."""

    def __init__(self, out, query, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                 partition_size=0, workspace=None, stream=None, new_key=None, new_value=None,
                 host_context_lens=None, write_cache=True, group_size=1):
        """With new_key/new_value: the fused append (write_cache) or the newest-token variant that
        leaves the cache to the caller (write_cache=False).  group_size > 1: the grouped decode
        (paged_attention_decode_grouped; no fused append)."""
        if group_size > 1 and new_key is not None:
            raise ValueError("the grouped decode has no fused append")
        self.group_size = int(group_size)
        hl, hp = _host_lens_ptr(host_context_lens)
        self._keep = (out, query, k_cache, v_cache, block_tables, context_lens, workspace, new_key, new_value, hl)
        self.args = _decode_args(out, query, k_cache, v_cache, block_tables, context_lens, max_context_len, scale,
                                 partition_size, workspace, hp)
        self.fused_args = None if new_key is None else _fused_args(self.args, new_key, new_value)
        self.write_cache = write_cache
        self.stream = _stream(stream)
        B, Hq, D = query.shape
        self.reduce_args = (out.data_ptr(), dtype_code(out.dtype), context_lens.data_ptr(), B, Hq, D,
                            int(max_context_len), int(partition_size), self.args[17], self.args[18])

    def __call__(self) -> None:
        if self.fused_args is not None:
            fn = lib.paged_attention_decode_append if self.write_cache else lib.paged_attention_decode_newest
            check(fn(*self.fused_args, self.stream))
        elif self.group_size > 1:
            check(lib.paged_attention_decode_grouped(*self.args[:20], self.group_size, self.stream))
        else:
            check(lib.paged_attention_decode(*self.args, self.stream))

    def partitions(self) -> None:
        if self.fused_args is not None:
            fn = (lib.paged_attention_decode_append_partitions if self.write_cache else
                  lib.paged_attention_decode_newest_partitions)
            check(fn(*self.fused_args, self.stream))
        else:
            check(lib.paged_attention_decode_partitions(*self.args, self.stream))

    def reduce(self) -> None:
        check(lib.paged_attention_decode_reduce(*self.reduce_args, self.stream))


class PreparedAppend:
    """paged_cache_append with its arguments marshalled once."""

    def __init__(self, k_cache, v_cache, key, value, slot_mapping, stream=None):
        _dev(k_cache, v_cache, key, value, slot_mapping)
        self._keep = (k_cache, v_cache, key, value, slot_mapping)
        N, H, D = cache_dims(k_cache, v_cache)
        bs = 16
        T = slot_mapping.numel()
        if key.dtype != k_cache.dtype or value.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype:
            raise TypeError("key, value and caches must share one dtype")
        if key.shape != (T, H, D) or value.shape != (T, H, D) or slot_mapping.dtype != torch.int32:
            raise ValueError("key/value must be [T][Hkv][D], slot_mapping int32 [T]")
        self.args = (k_cache.data_ptr(), v_cache.data_ptr(), key.data_ptr(), value.data_ptr(), 0, 0,
                     slot_mapping.data_ptr(), T, H, D, bs, N, dtype_code(k_cache.dtype))
        self.stream = _stream(stream)

    def __call__(self) -> None:
        check(lib.paged_cache_append(*self.args, self.stream))


# ---- FP8 (E4M3) cache: code tiles uint8 k and v [N][Hkv][16 * D] (stored orders of
# ---- include/pagedkv.h, flat for the same reason as kv_cache); scales fp32 [N][Hkv][16] for K and
# ---- for V (entry [b, h, t] is slot t's scale).
def fp8_cache(num_blocks: int, num_kv_heads: int, head_dim: int, device="cuda"):
    """Allocate (k, v, k_scale, v_scale) of an fp8 cache, filled with the NaN code / NaN scales."""
    k = torch.full((num_blocks, num_kv_heads, 16 * head_dim), 0x7F, dtype=torch.uint8, device=device)
    v = torch.full_like(k, 0x7F)
    ks = torch.full((num_blocks, num_kv_heads, 16), float("nan"), dtype=torch.float32, device=device)
    vs = torch.full_like(ks, float("nan"))
    return k, v, ks, vs


def _fp8_shapes(k_cache, v_cache, k_scale, v_scale):
    _dev(k_cache, v_cache, k_scale, v_scale)
    N, H, D = cache_dims(k_cache, v_cache)
    bs = 16
    if k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
        raise TypeError("fp8 caches are uint8 tensors of E4M3 codes")
    if tuple(k_scale.shape) != (N, H, bs) or k_scale.shape != v_scale.shape:
        raise ValueError("fp8 scales must be [N][Hkv][16]")
    if k_scale.dtype != torch.float32 or v_scale.dtype != torch.float32:
        raise TypeError("fp8 scales are float32")
    return N, H, bs, D


def paged_cache_append_fp8(k_cache, v_cache, k_scale, v_scale, key, value, slot_mapping, stream=None) -> None:
    """Quantise key/value [T][Hkv][D] (fp32/fp16/bf16) into their slots."""
    N, H, bs, D = _fp8_shapes(k_cache, v_cache, k_scale, v_scale)
    _dev(key, value, slot_mapping)
    if key.dtype != value.dtype:
        raise TypeError("key and value must share one dtype")
    if slot_mapping.dtype != torch.int32:
        raise TypeError("slot_mapping must be int32")
    T = slot_mapping.numel()
    if key.shape != (T, H, D) or value.shape != (T, H, D):
        raise ValueError("key/value must be [T][Hkv][D]")
    check(lib.paged_cache_append_fp8(k_cache.data_ptr(), v_cache.data_ptr(), k_scale.data_ptr(), v_scale.data_ptr(),
                                     key.data_ptr(), value.data_ptr(), 0, 0, slot_mapping.data_ptr(), T, H, D, bs, N,
                                     dtype_code(key.dtype), _stream(stream)))


def paged_cache_copy_blocks_fp8(k_cache, v_cache, k_scale, v_scale, src_dst, stream=None) -> None:
    N, H, bs, D = _fp8_shapes(k_cache, v_cache, k_scale, v_scale)
    _dev(src_dst)
    if src_dst.dtype != torch.int32 or src_dst.dim() != 2 or src_dst.shape[1] != 2:
        raise ValueError("src_dst must be int32 [n][2]")
    check(lib.paged_cache_copy_blocks_fp8(k_cache.data_ptr(), v_cache.data_ptr(), k_scale.data_ptr(),
                                          v_scale.data_ptr(), src_dst.data_ptr(), src_dst.shape[0], H, D, bs, N,
                                          _stream(stream)))


def _fp8_decode_args(out, query, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, max_context_len,
                     scale, partition_size, workspace, host_ptr):
    N, Hkv, bs, D = _fp8_shapes(k_cache, v_cache, k_scale, v_scale)
    _dev(out, query, block_tables, context_lens)
    B, Hq, Dq = query.shape
    if Dq != D or out.shape != query.shape:
        raise ValueError("query/out must be [B][Hq][head_dim]")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise TypeError("block_tables and context_lens must be int32")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.shape != (B,):
        raise ValueError("block_tables must be [B][max_blocks], context_lens [B]")
    ws_ptr, ws_bytes = (0, 0) if workspace is None else (workspace.data_ptr(), workspace.numel() * workspace.element_size())
    return (out.data_ptr(), dtype_code(out.dtype), query.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            k_scale.data_ptr(), v_scale.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(), B, Hq, Hkv, D,
            bs, block_tables.shape[1], N, int(max_context_len), float(scale), int(partition_size), ws_ptr, ws_bytes,
            dtype_code(query.dtype), host_ptr)


def paged_attention_decode_fp8(out, query, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                               max_context_len, scale, partition_size=0, workspace=None, stream=None,
                               host_context_lens=None) -> None:
    """Decode attention over an fp8 cache; query bf16/fp16 [B][Hq][D]; out fp32 or the query dtype."""
    hl, hp = _host_lens_ptr(host_context_lens)
    args = _fp8_decode_args(out, query, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                            max_context_len, scale, partition_size, workspace, hp)
    check(lib.paged_attention_decode_fp8(*args, _stream(stream)))


def paged_attention_decode_grouped_fp8(out, query, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                                       max_context_len, scale, group_size, partition_size=0, workspace=None,
                                       stream=None) -> None:
    """paged_attention_decode_fp8 with sequences group_size to a workgroup, so that blocks their
    tables share are read once; bit for bit paged_attention_decode_fp8's output."""
    args = _fp8_decode_args(out, query, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                            max_context_len, scale, partition_size, workspace, None)
    check(lib.paged_attention_decode_grouped_fp8(*args[:22], int(group_size), _stream(stream)))


def _fp8_prefill_args(out, query, k_cache, v_cache, k_scale, v_scale, block_table, ctx_start, scale):
    N, Hkv, bs, D = _fp8_shapes(k_cache, v_cache, k_scale, v_scale)
    _dev(out, query, block_table)
    if query.dim() != 3 or out.shape != query.shape or query.shape[2] != D:
        raise ValueError("query and out must be [C][Hq][head_dim]")
    C, Hq, _ = query.shape
    if block_table.dtype != torch.int32:
        raise TypeError("block_table must be int32")
    if block_table.numel() * bs < ctx_start + C:
        raise ValueError("block_table too short for ctx_start + C")
    return (out.data_ptr(), dtype_code(out.dtype), query.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            k_scale.data_ptr(), v_scale.data_ptr(), block_table.data_ptr(), int(ctx_start), C, Hq, Hkv, D, bs, N,
            float(scale), dtype_code(query.dtype))


def paged_attention_prefill_chunk_fp8(out, query, k_cache, v_cache, k_scale, v_scale, block_table, ctx_start, scale,
                                      stream=None) -> None:
    """Prefill chunk over an fp8 cache; query bf16/fp16 [C][Hq][D]; out fp32 or the query dtype."""
    check(lib.paged_attention_prefill_chunk_fp8(*_fp8_prefill_args(out, query, k_cache, v_cache, k_scale, v_scale,
                                                                   block_table, ctx_start, scale), _stream(stream)))


class PreparedPrefillFp8:
    """paged_attention_prefill_chunk_fp8 with its arguments marshalled once."""

    def __init__(self, out, query, k_cache, v_cache, k_scale, v_scale, block_table, ctx_start, scale, stream=None):
        self._keep = (out, query, k_cache, v_cache, k_scale, v_scale, block_table)
        self.args = _fp8_prefill_args(out, query, k_cache, v_cache, k_scale, v_scale, block_table, ctx_start, scale)
        self.stream = _stream(stream)

    def __call__(self) -> None:
        check(lib.paged_attention_prefill_chunk_fp8(*self.args, self.stream))


def _fp8_fused_args(args, new_key, new_value):
    """Argument tuple of paged_attention_decode_append_fp8 from a _fp8_decode_args tuple."""
    _dev(new_key, new_value)
    B, Hkv, D = args[9], args[11], args[12]
    for t in (new_key, new_value):
        if tuple(t.shape) != (B, Hkv, D) or dtype_code(t.dtype) != args[21]:
            raise ValueError("new_key/new_value must be [B][Hkv][D] of the query dtype")
    return args[:3] + (new_key.data_ptr(), new_value.data_ptr()) + args[3:]


def paged_attention_decode_append_fp8(out, query, new_key, new_value, k_cache, v_cache, k_scale, v_scale,
                                      block_tables, context_lens, max_context_len, scale, partition_size=0,
                                      workspace=None, stream=None, host_context_lens=None) -> None:
    """One decode step over an fp8 cache with the quantising append fused in: token
    context_lens[b] - 1 of every sequence (new_key/new_value [B][Hkv][D], the query's dtype) is
    quantised into its slot and attended over."""
    hl, hp = _host_lens_ptr(host_context_lens)
    args = _fp8_decode_args(out, query, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                            max_context_len, scale, partition_size, workspace, hp)
    check(lib.paged_attention_decode_append_fp8(*_fp8_fused_args(args, new_key, new_value), _stream(stream)))


class PreparedDecodeFp8:
    """paged_attention_decode_fp8 with its arguments marshalled once (partitions / reduce separately);
    with new_key/new_value, calling it runs paged_attention_decode_append_fp8 instead."""

    def __init__(self, out, query, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, max_context_len,
                 scale, partition_size=0, workspace=None, stream=None, host_context_lens=None, new_key=None,
                 new_value=None):
        self._hl, hp = _host_lens_ptr(host_context_lens)
        self._keep = (out, query, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, workspace,
                      new_key, new_value)
        self.args = _fp8_decode_args(out, query, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                                     max_context_len, scale, partition_size, workspace, hp)
        self.fused_args = None if new_key is None else _fp8_fused_args(self.args, new_key, new_value)
        B, Hq, D = query.shape
        ws_ptr, ws_bytes = self.args[19], self.args[20]
        self.reduce_args = (out.data_ptr(), dtype_code(out.dtype), context_lens.data_ptr(), B, Hq, D,
                            int(max_context_len), int(partition_size), ws_ptr, ws_bytes)
        self.stream = _stream(stream)

    def __call__(self) -> None:
        if self.fused_args is not None:
            check(lib.paged_attention_decode_append_fp8(*self.fused_args, self.stream))
        else:
            check(lib.paged_attention_decode_fp8(*self.args, self.stream))

    def partitions(self) -> None:
        check(lib.paged_attention_decode_fp8_partitions(*self.args, self.stream))

    def reduce(self) -> None:
        check(lib.paged_attention_decode_reduce(*self.reduce_args, self.stream))


class PreparedAppendFp8:
    """paged_cache_append_fp8 with its arguments marshalled once."""

    def __init__(self, k_cache, v_cache, k_scale, v_scale, key, value, slot_mapping, stream=None):
        N, H, bs, D = _fp8_shapes(k_cache, v_cache, k_scale, v_scale)
        _dev(key, value, slot_mapping)
        T = slot_mapping.numel()
        if key.shape != (T, H, D) or value.shape != (T, H, D) or slot_mapping.dtype != torch.int32:
            raise ValueError("key/value must be [T][Hkv][D], slot_mapping int32 [T]")
        self._keep = (k_cache, v_cache, k_scale, v_scale, key, value, slot_mapping)
        self.args = (k_cache.data_ptr(), v_cache.data_ptr(), k_scale.data_ptr(), v_scale.data_ptr(), key.data_ptr(),
                     value.data_ptr(), 0, 0, slot_mapping.data_ptr(), T, H, D, bs, N, dtype_code(key.dtype))
        self.stream = _stream(stream)

    def __call__(self) -> None:
        check(lib.paged_cache_append_fp8(*self.args, self.stream))


def _mixed_args(dec_out, dec_query, dec_tables, dec_lens, dec_max_context_len, pre_out, pre_query, pre_tables,
                ctx_starts, chunk_lens, k_cache, v_cache, scale, host_dec_lens, dec_partition_size=0, dec_group_size=1,
                workspace=None, k_scale=None, v_scale=None):
    """Every shape and dtype is checked before the tensors' device (so a mismatch is reported as
    such), and all of it before the launch.  With k_scale / v_scale: the fp8 cache and the argument
    order of paged_attention_mixed_fp8 (queries bf16 or fp16)."""
    fp8 = k_scale is not None or v_scale is not None
    if fp8:
        if k_scale is None or v_scale is None:
            raise ValueError("an fp8 cache needs both k_scale and v_scale")
        if dec_group_size != 1:
            raise ValueError("the fp8 mixed launch has no grouped decode")
        N, Hkv, bs, D = _fp8_shapes(k_cache, v_cache, k_scale, v_scale)
        qs = [t for t in (dec_query, pre_query) if t is not None and t.numel()]
        qdt = qs[0].dtype if qs else torch.bfloat16
        if qdt not in (torch.bfloat16, torch.float16) or any(t.dtype != qdt for t in qs):
            raise TypeError("fp8 mixed queries must share one dtype, bf16 or fp16")
        dtype = dtype_code(qdt)
        cache_dt = qdt  # the dtype the query checks below compare against
    else:
        N, Hkv, D = cache_dims(k_cache, v_cache)
        bs = 16
        if v_cache.dtype != k_cache.dtype:
            raise TypeError("k_cache and v_cache must share one dtype")
        dtype = dtype_code(k_cache.dtype)
        cache_dt = k_cache.dtype
    B = 0 if dec_query is None else dec_query.shape[0]
    S = len(chunk_lens)
    Hq = out_dtype = None
    if B:
        if dec_query.dim() != 3 or dec_query.shape[2] != D:
            raise ValueError("dec_query must be [B][Hq][head_dim]")
        if tuple(dec_out.shape) != tuple(dec_query.shape):
            raise ValueError("dec_out must have dec_query's shape [B][Hq][D]")
        if dec_query.dtype != cache_dt:
            raise TypeError("dec_query must have the cache dtype")
        if dec_tables.dtype != torch.int32 or dec_lens.dtype != torch.int32:
            raise TypeError("decode tables and lens must be int32")
        if dec_tables.dim() != 2 or dec_tables.shape[0] != B or tuple(dec_lens.shape) != (B,):
            raise ValueError("decode tables must be [B][max_blocks] and lens [B]")
        Hq = dec_query.shape[1]
        out_dtype = dec_out.dtype
    if S:
        if pre_query.dim() != 3 or pre_query.shape[2] != D:
            raise ValueError("pre_query must be [rows][Hq][head_dim]")
        if pre_query.dtype != cache_dt:
            raise TypeError("pre_query must have the cache dtype")
        if pre_tables.dtype != torch.int32 or pre_tables.dim() != 2 or pre_tables.shape[0] != S:
            raise ValueError("prefill tables must be int32 [num_chunks][max_blocks]")
        if pre_query.shape[0] != int(sum(chunk_lens)) or tuple(pre_out.shape) != tuple(pre_query.shape):
            raise ValueError("pre_query / pre_out must hold sum(chunk_lens) rows")
        if Hq is not None and pre_query.shape[1] != Hq:
            raise ValueError("decode and prefill queries must have the same number of heads")
        if out_dtype is not None and pre_out.dtype != out_dtype:
            raise TypeError("dec_out and pre_out must share one dtype (one out_dtype per launch)")
        Hq = pre_query.shape[1]
        out_dtype = pre_out.dtype
    if not B and not S:
        return None
    starts = np.ascontiguousarray(np.asarray(ctx_starts, dtype=np.int32))
    lens = np.ascontiguousarray(np.asarray(chunk_lens, dtype=np.int32))
    if len(starts) != S:
        raise ValueError("ctx_starts and chunk_lens must have one entry per chunk")
    _dev(k_cache, v_cache, *((k_scale, v_scale) if fp8 else ()), *((dec_out, dec_query, dec_tables, dec_lens) if B else ()),
         *((pre_out, pre_query, pre_tables) if S else ()))
    hl, hp = _host_lens_ptr(host_dec_lens)
    keep = (starts, lens, hl)
    if workspace is not None:
        _dev(workspace)
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (workspace.data_ptr(),
                                                            workspace.numel() * workspace.element_size())
    dec = (dec_out.data_ptr() if B else None, dec_query.data_ptr() if B else None,
           dec_tables.data_ptr() if B else None, dec_lens.data_ptr() if B else None, B,
           dec_tables.shape[1] if B else 0, int(dec_max_context_len) if B else 0, hp, int(dec_partition_size))
    pre = (pre_out.data_ptr() if S else None, pre_query.data_ptr() if S else None,
           pre_tables.data_ptr() if S else None, pre_tables.shape[1] if S else 0,
           starts.ctypes.data if S else None, lens.ctypes.data if S else None, S, dtype_code(out_dtype))
    if fp8:
        args = dec + (ws_ptr, ws_bytes) + pre + (k_cache.data_ptr(), v_cache.data_ptr(), k_scale.data_ptr(),
                                                 v_scale.data_ptr(), Hq, Hkv, D, bs, N, float(scale), dtype)
    else:
        args = dec + (int(dec_group_size), ws_ptr, ws_bytes) + pre + (k_cache.data_ptr(), v_cache.data_ptr(), Hq, Hkv,
                                                                      D, bs, N, float(scale), dtype)
    return args, keep


def paged_attention_mixed(dec_out, dec_query, dec_tables, dec_lens, dec_max_context_len, pre_out, pre_query,
                          pre_tables, ctx_starts, chunk_lens, k_cache, v_cache, scale, stream=None,
                          host_dec_lens=None, dec_partition_size=0, dec_group_size=1, workspace=None) -> None:
    """One launch (+ the split-K merge when dec_partition_size > 0): decode of a batch (grouped
    dec_group_size sequences to a workgroup when > 1) + causal attention of prefill chunks (rows
    packed in pre_query/pre_out; chunk i at positions ctx_starts[i] .., table row i of pre_tables)."""
    r = _mixed_args(dec_out, dec_query, dec_tables, dec_lens, dec_max_context_len, pre_out, pre_query, pre_tables,
                    ctx_starts, chunk_lens, k_cache, v_cache, scale, host_dec_lens, dec_partition_size,
                    dec_group_size, workspace)
    if r is None:
        return
    args, keep = r
    check(lib.paged_attention_mixed(*args, _stream(stream)))


def paged_attention_mixed_fp8(dec_out, dec_query, dec_tables, dec_lens, dec_max_context_len, pre_out, pre_query,
                              pre_tables, ctx_starts, chunk_lens, k_cache, v_cache, k_scale, v_scale, scale,
                              stream=None, host_dec_lens=None, dec_partition_size=0, workspace=None) -> None:
    """paged_attention_mixed over an fp8 cache (codes + per-slot scales); bf16/fp16 queries."""
    r = _mixed_args(dec_out, dec_query, dec_tables, dec_lens, dec_max_context_len, pre_out, pre_query, pre_tables,
                    ctx_starts, chunk_lens, k_cache, v_cache, scale, host_dec_lens, dec_partition_size, 1,
                    workspace, k_scale, v_scale)
    if r is None:
        return
    args, keep = r
    check(lib.paged_attention_mixed_fp8(*args, _stream(stream)))


class PreparedMixed:
    """paged_attention_mixed with its arguments marshalled once."""

    def __init__(self, *a, stream=None, host_dec_lens=None, dec_partition_size=0, dec_group_size=1,
                 workspace=None):
        self._tensors = (a, workspace)
        r = _mixed_args(*a, host_dec_lens=host_dec_lens, dec_partition_size=dec_partition_size,
                        dec_group_size=dec_group_size, workspace=workspace)
        self.args, self._keep = r
        self.stream = _stream(stream)

    def __call__(self) -> None:
        check(lib.paged_attention_mixed(*self.args, self.stream))
