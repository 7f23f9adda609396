"""paged_kv_cache_404_amd - paged KV-cache decode attention for AMD MI355X (gfx950).

A C-ABI library (libpagedkv.so, declared in include/pagedkv.h) holds the whole hot path: the host
block pool and builders (C++) and the HIP kernels (cache append, copy-on-write block copy, paged
decode attention with split-K, chunked-prefill causal attention).  This package is a thin binding:
``pool.BlockPool`` over the pool calls and ``ops`` over the device calls (torch tensors for device
memory and streams).  Importing it fails when the library is not built; there is no fallback.
"""
from ._lib import (EXPORTED, PKV_BF16, PKV_EHIP, PKV_EINVAL, PKV_ENOMEM, PKV_EUNSUPPORTED, PKV_F16, PKV_F32,  # noqa: F401
                   PKV_OK, PKV_SINGLE_PASS_ADAPTIVE, LIB_PATH, OutOfBlocksError, PagedKVError, last_error, lib)
from .pool import BlockPool  # noqa: F401


def version() -> int:
    return int(lib.pkv_version())
