"""ctypes declarations for libpagedkv.so (the C ABI in include/pagedkv.h).

Loading fails loudly when the library has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedkv.so")

PKV_OK = 0
PKV_EINVAL = -1
PKV_ENOMEM = -2
PKV_EUNSUPPORTED = -3
PKV_EHIP = -4

PKV_F32 = 0
PKV_F16 = 1
PKV_BF16 = 2

# partition_size value: a batch-adaptive single pass (faster on short contexts, not batch invariant).
PKV_SINGLE_PASS_ADAPTIVE = -1

# Size of the static device scratch behind paged_attention_decode_noalloc, per GPU.
PKV_NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024


class PagedKVError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[status {status}] {message}")
        self.status = status


class OutOfBlocksError(PagedKVError):
    """The block pool cannot cover an allocation (PKV_ENOMEM)."""


# torch bundles its own HIP runtime with the same SONAME as ROCm's.  Loading torch first makes the
# library bind to that runtime instead of pulling a second copy into the process (two runtimes in
# one process do not share devices, streams or memory).
import torch  # noqa: E402,F401

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python paged_kv_cache_404_amd/build.py` (hipcc, gfx950). "
        "This package has no non-HIP fallback.")

lib = C.CDLL(LIB_PATH)

_i32, _i64, _f32, _vp, _sz = C.c_int32, C.c_int64, C.c_float, C.c_void_p, C.c_size_t
_pi32 = C.POINTER(C.c_int32)
_pool_p = C.c_void_p

_SIGS = {
    "pkv_last_error": (C.c_char_p, []),
    "pkv_version": (_i32, []),
    "paged_cache_append": (C.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp]),
    "paged_cache_copy_blocks": (C.c_int, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp]),
    "paged_attention_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "paged_attention_decode": (C.c_int, [_vp, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                         _i32, _i32, _f32, _i32, _vp, _sz, _i32, _vp, _vp]),
    "paged_attention_decode_grouped": (C.c_int, [_vp, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                                 _i32, _i32, _i32, _f32, _i32, _vp, _sz, _i32, _i32, _vp]),
    "paged_attention_decode_noalloc": (C.c_int, [_vp, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                                 _i32, _i32, _i32, _f32, _i32, _i32, _vp, _vp]),
    "paged_attention_decode_partitions": (C.c_int, [_vp, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                                    _i32, _i32, _i32, _f32, _i32, _vp, _sz, _i32, _vp, _vp]),
    "paged_attention_decode_reduce": (C.c_int, [_vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _sz, _vp]),
    "paged_attention_decode_append": (C.c_int, [_vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                                _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz, _i32, _vp, _vp]),
    "paged_attention_decode_append_partitions": (C.c_int, [_vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                                           _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz,
                                                           _i32, _vp, _vp]),
    "paged_attention_decode_newest": (C.c_int, [_vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                                _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz, _i32, _vp, _vp]),
    "paged_attention_decode_newest_partitions": (C.c_int, [_vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                                           _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz,
                                                           _i32, _vp, _vp]),
    "paged_attention_prefill_chunk": (C.c_int, [_vp, _i32, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                                _i32, _f32, _i32, _vp]),
    "paged_attention_mixed": (C.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _i32, _i32, _vp, _sz, _vp, _vp, _vp,
                                        _i32, _vp, _vp, _i32, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _f32, _i32,
                                        _vp]),
    "paged_attention_mixed_fp8": (C.c_int, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _i32, _vp, _sz, _vp, _vp,
                                            _vp, _i32, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                            _i32, _i32, _f32, _i32, _vp]),
    "paged_cache_append_fp8": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _vp, _i32, _i32, _i32, _i32,
                                         _i32, _i32, _vp]),
    "paged_cache_copy_blocks_fp8": (C.c_int, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp]),
    "paged_check_inputs": (C.c_int, [_vp, _vp, _i32, _i32, _i32, _vp, _i32, _i32, _i32, _vp, _vp]),
    "paged_probe_stream_read": (C.c_int, [_vp, _sz, _vp, _i32, _vp]),
    "paged_attention_prefill_chunk_fp8": (C.c_int, [_vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                                    _i32, _i32, _i32, _f32, _i32, _vp]),
    "paged_attention_decode_fp8": (C.c_int, [_vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                             _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz, _i32, _vp, _vp]),
    "paged_attention_decode_grouped_fp8": (C.c_int, [_vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                                     _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz, _i32,
                                                     _i32, _vp]),
    "paged_attention_decode_fp8_partitions": (C.c_int, [_vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                                        _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz,
                                                        _i32, _vp, _vp]),
    "paged_attention_decode_append_fp8": (C.c_int, [_vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                                                    _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _i32, _vp, _sz,
                                                    _i32, _vp, _vp]),
    "pkv_pool_create": (C.c_int, [_i32, _i32, _vp, C.POINTER(_pool_p)]),
    "pkv_pool_destroy": (None, [_pool_p]),
    "pkv_pool_num_free": (C.c_int, [_pool_p, _vp]),
    "pkv_pool_free_list": (C.c_int, [_pool_p, _vp, _i32, _vp]),
    "pkv_pool_refcount": (C.c_int, [_pool_p, _i32, _vp]),
    "pkv_seq_new": (C.c_int, [_pool_p, _vp]),
    "pkv_seq_fork": (C.c_int, [_pool_p, _i32, _vp]),
    "pkv_seq_blocks_needed": (C.c_int, [_pool_p, _i32, _i32, _vp]),
    "pkv_seq_append": (C.c_int, [_pool_p, _i32, _i32, _vp, _vp, _vp]),
    "pkv_seqs_append": (C.c_int, [_pool_p, _vp, _vp, _i32, _vp, _vp, _vp, _vp]),
    "pkv_seq_free": (C.c_int, [_pool_p, _i32]),
    "pkv_seq_len": (C.c_int, [_pool_p, _i32, _vp]),
    "pkv_seq_num_blocks": (C.c_int, [_pool_p, _i32, _vp]),
    "pkv_build_block_tables": (C.c_int, [_pool_p, _vp, _i32, _i32, _vp, _vp]),
    "pkv_build_slot_mapping": (C.c_int, [_pool_p, _vp, _vp, _vp, _i32, _vp]),
    "pkv_prefix_insert": (C.c_int, [_pool_p, _i32, _vp, _i32, _vp]),
    "pkv_prefix_lookup": (C.c_int, [_pool_p, _vp, _i32, _vp, _vp]),
    "pkv_prefix_evictable": (C.c_int, [_pool_p, _vp, _i32, _vp]),
    "pkv_prefix_num_registered": (C.c_int, [_pool_p, _vp]),
}

for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGS)


def last_error() -> str:
    m = lib.pkv_last_error()
    return m.decode() if m else ""


def check(status: int) -> None:
    if status == PKV_OK:
        return
    msg = last_error()
    if status == PKV_ENOMEM:
        raise OutOfBlocksError(status, msg)
    raise PagedKVError(status, msg)
