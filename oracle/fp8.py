"""FP8 K/V cache model.  TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

[Notes] "Continuous batching and PagedAttention: serving many users from one GPU", "Memory, not
compute, caps the batch": the cache, not the arithmetic, limits how many sequences run at once,
and a quantised cache multiplies the tokens that fit.  The format here is the 8-bit float E4M3 of
the OCP 8-bit Floating Point Specification (OFP8), which the pages do not name:
sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent 0 holds the subnormals m * 2^-9;
exponent 15 with mantissa 7 is NaN; there are no infinities; the largest finite value is 448.

Quantisation of one (token, KV head) row x of head_dim values (x exact in fp32):
    amax = max_i |x_i|
    s    = fp32(amax / 448)                   (the stored scale)
    inv  = fp32(448 / amax), or 0 when amax = 0
    code = E4M3 round-to-nearest-even of fp32(x_i * inv)
and the value the cache stands for is decode(code) * s.  |x_i * inv| <= 448 (1 + 2^-23) rounds to at
most 448, so no code saturates.  K and V rows are quantised separately; each (block, head, slot)
has its own K scale and V scale.

Layout (the library's, reproduced here independently from its description): a K tile of one
(block, head) is 16 tokens x head_dim bytes with byte (t, d) at
    ((d // 64) * 2 + (t // 4) % 2) * 512 + ((t // 8) * 4 + t % 4) * 64 + d % 64
and a V tile is dimension-major, byte (t, d) at d * 16 + t.  Scales are fp32 [block][head][slot].
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
NAN_CODE = 0x7F


def e4m3_decode(codes) -> np.ndarray:
    """Exact value of each code (NaN for the two NaN codes), as fp64."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def e4m3_encode(x) -> np.ndarray:
    """Round each value to the nearest E4M3 value, ties to the even code; |x| must not exceed
    448 (1 + 2^-23) (so that nothing rounds past the largest finite value)."""
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any() or (np.abs(x) >= 464.0).any():
        raise ValueError("e4m3_encode: NaN or |x| >= 464 (outside the rounding range of 448)")
    a = np.abs(x)
    sign = np.signbit(x).astype(np.int64) << 7
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    sub = a < 2.0 ** -6
    # subnormal grid: steps of 2^-9; normal grid of binade e: steps of 2^(e - 3)
    step_exp = np.where(sub, -9.0, e - 3.0)
    q = np.rint(a / np.exp2(step_exp))  # exact scaling by a power of two; rint = half to even
    code = np.where(sub, q, (e + 7.0) * 8.0 + (q - 8.0)).astype(np.int64)  # q = 16 carries into e + 1
    return (sign | code).astype(np.uint8)


def quantize_rows(x32: np.ndarray):
    """x32: fp32 [..., D] rows.  Returns (codes uint8 [..., D], scales fp32 [...])."""
    x32 = np.asarray(x32, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=-1)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(amax > 0, np.float32(E4M3_MAX) / np.where(amax > 0, amax, np.float32(1)), 0).astype(np.float32)
    y = (x32 * inv[..., None]).astype(np.float32)
    return e4m3_encode(y), s


def k_byte_offset(t: int, d: int) -> int:
    return ((d // 64) * 2 + (t // 4) % 2) * 512 + ((t // 8) * 4 + t % 4) * 64 + d % 64


class Fp8CacheModel:
    """Pool of fp8 K/V codes with per-(block, head, slot) scales, filled by appends."""

    dtype = "fp8"

    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int, block_size: int = 16):
        self.N, self.H, self.D, self.bs = num_blocks, num_kv_heads, head_dim, block_size
        self.k = np.full((self.N, self.H, self.bs, self.D), NAN_CODE, dtype=np.uint8)
        self.v = np.full((self.N, self.H, self.D, self.bs), NAN_CODE, dtype=np.uint8)
        self.k_scale = np.full((self.N, self.H, self.bs), np.nan, dtype=np.float32)
        self.v_scale = np.full((self.N, self.H, self.bs), np.nan, dtype=np.float32)

    def append(self, key32: np.ndarray, value32: np.ndarray, slots) -> None:
        """key32/value32: fp32 [T][H][D] (the input rows widened exactly); slot -1 = skip."""
        kc, ks = quantize_rows(key32)
        vc, vs = quantize_rows(value32)
        for t, slot in enumerate(slots):
            slot = int(slot)
            if slot < 0:
                continue
            blk, off = divmod(slot, self.bs)
            self.k[blk, :, off, :] = kc[t]
            self.v[blk, :, :, off] = vc[t]
            self.k_scale[blk, :, off] = ks[t]
            self.v_scale[blk, :, off] = vs[t]

    def copy_blocks(self, pairs) -> None:
        for src, dst in pairs:
            self.k[dst] = self.k[src]
            self.v[dst] = self.v[src]
            self.k_scale[dst] = self.k_scale[src]
            self.v_scale[dst] = self.v_scale[src]

    def dequant_kv(self, blocks):
        """fp64 K [nb][H][bs][D] and V [nb][H][D][bs] of the given blocks: code value * scale."""
        k = e4m3_decode(self.k[blocks]) * self.k_scale[blocks][..., None].astype(np.float64)
        v = e4m3_decode(self.v[blocks]) * self.v_scale[blocks][:, :, None, :].astype(np.float64)
        return k, v

    def v_physical(self, blocks=slice(None)) -> np.ndarray:
        """V codes in the library's tile order ([D][16] per tile): [n][H][16 * D] bytes."""
        v = self.v[blocks]
        return np.ascontiguousarray(v).reshape(v.shape[0], self.H, self.D * self.bs)

    def k_physical(self, blocks=slice(None)) -> np.ndarray:
        """K codes in the library's tile order: [n][H][16 * D] bytes."""
        k = self.k[blocks]
        n = k.shape[0]
        out = np.empty((n, self.H, self.bs * self.D), dtype=np.uint8)
        for t in range(self.bs):
            for d in range(self.D):
                out[:, :, k_byte_offset(t, d)] = k[:, :, t, d]
        return out
