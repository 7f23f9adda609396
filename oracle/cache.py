"""Oracle model of the paged K/V cache bytes.  TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

[Serving] The Build, Step 4 keeps every page in one big tensor indexed by physical page
id and writes token ``pos`` of a sequence at (page, pos % block_size).  This library
stores one layer's K and V as two such tensors.  Layout (a fixed part of the library's
interface, restated here independently):

    V: [num_blocks][num_kv_heads][tile], one tile per (block, head) nested
       [token half t // 8][head_dim][8 tokens t % 8]
    K: [num_blocks][num_kv_heads][tile], one tile of block_size (16) tokens x head_dim
       elements per (block, head), in 16-byte chunks (E = 16 / element size elements each).
       Number the tokens t = 8*hi + 4*set + low and the chunks of a token's head vector
       c = 4*cq + cr; the tile stores the chunks in the nested order
       [cq][set][cr][hi][low], each chunk's E elements in order.

``self.k`` holds K in the logical order [num_blocks][num_kv_heads][block_size][head_dim] and
``self.v`` holds V as [num_blocks][num_kv_heads][head_dim][block_size] (what attention reads);
``k_physical()`` and ``v_physical()`` rearrange them into the stored orders above, which is what
the library's device tensors must hold byte for byte.

Slot ``s`` means block ``s // block_size``, offset ``s % block_size``; slot -1 is skipped.
Values are held as raw storage bits (uint16 for bf16/fp16, uint32 for fp32), so append and
block copy are byte copies with no arithmetic.
"""
from __future__ import annotations

import numpy as np

_NAN = {"bf16": 0x7FC0, "f16": 0x7E00, "f32": 0x7FC00000}
_NP = {"bf16": np.uint16, "f16": np.uint16, "f32": np.uint32}


class CacheModel:
    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int, dtype: str,
                 block_size: int = 16, fill_nan: bool = True):
        self.N, self.H, self.D, self.bs, self.dtype = num_blocks, num_kv_heads, head_dim, block_size, dtype
        t = _NP[dtype]
        fill = _NAN[dtype] if fill_nan else 0
        self.k = np.full((num_blocks, num_kv_heads, block_size, head_dim), fill, dtype=t)
        self.v = np.full((num_blocks, num_kv_heads, head_dim, block_size), fill, dtype=t)

    def append(self, key_bits: np.ndarray, value_bits: np.ndarray, slots) -> None:
        """key/value: [T][num_kv_heads][head_dim] bits; token t goes to slots[t] (skip -1)."""
        for t, s in enumerate(slots):
            s = int(s)
            if s < 0:
                continue
            blk, off = divmod(s, self.bs)
            if blk >= self.N:
                raise IndexError("slot outside the pool")
            self.k[blk, :, off, :] = key_bits[t]  # [H][D] -> every head's row `off`
            self.v[blk, :, :, off] = value_bits[t]  # [H][D] -> every head's column `off`

    def copy_blocks(self, pairs) -> None:
        """Whole-block copy of K and V for each (src, dst), in order."""
        for src, dst in pairs:
            self.k[dst] = self.k[src]
            self.v[dst] = self.v[src]

    def k_physical(self, blocks=slice(None)) -> np.ndarray:
        """K of the given blocks in stored byte order: [n][num_kv_heads][block_size * head_dim]."""
        k = self.k[blocks]
        n, H, bs, D = k.shape
        E = 16 // k.dtype.itemsize
        if bs != 16 or D % (4 * E):
            raise ValueError("the K tile order needs 16-token blocks and head_dim * elem_size % 64 == 0")
        # token axis -> (hi, set, low); dim axis -> (cq, cr, e)
        t = k.reshape(n, H, 2, 2, 4, D // (4 * E), 4, E)
        # stored order [cq][set][cr][hi][low][e]
        return np.ascontiguousarray(t.transpose(0, 1, 5, 3, 6, 2, 4, 7)).reshape(n, H, bs * D)

    def v_physical(self, blocks=slice(None)) -> np.ndarray:
        """V of the given blocks in stored order: per (block, head) the token halves, then the
        dimensions, then 8 tokens ([bs / 8][D][8]); returned as [n][num_kv_heads][block_size * head_dim]."""
        v = self.v[blocks]  # [n][H][D][bs]
        n, H, D, bs = v.shape
        if bs != 16:
            raise ValueError("the V tile order needs 16-token blocks")
        return np.ascontiguousarray(v.reshape(n, H, D, 2, 8).transpose(0, 1, 3, 2, 4)).reshape(n, H, bs * D)

    def token_k(self, slot: int) -> np.ndarray:
        blk, off = divmod(int(slot), self.bs)
        return self.k[blk, :, off, :]

    def token_v(self, slot: int) -> np.ndarray:
        blk, off = divmod(int(slot), self.bs)
        return self.v[blk, :, :, off]
