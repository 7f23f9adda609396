// Cache append (slot scatter) and whole-block copy-on-write copy.
//
// [Serving] "Production Serving: Continuous Batching and PagedAttention", The Build, Step 4:
// token pos of a sequence is stored at (page, pos % block_size) of one big tensor indexed by
// physical page id.  Here the slot of every token is computed on the host by the block pool, so
// the kernels only move bytes.  Layout: K [N][Hkv][tile] with each token's head vector cut into
// 16-byte chunks placed in the matrix-core tile order of k_chunk_pos (16-byte stores), V
// [N][Hkv][bs / 8][D][8] (per (block, head): token half, dimension, 8 tokens; a token is written
// element by element, its 8 dimensions of one chunk into one 128-byte line at bf16).
// Copy-on-write ([Chapter] "PagedAttention: KV cache memory"): a shared block that a sequence is
// about to write is first copied whole.
#include "device.h"

namespace pkv {
namespace {

// A workgroup writes one head of a window of TW = 256 / chunks consecutive input tokens (16 at
// D = 128 bf16), one thread per (token, 16-byte chunk of the head vector).  The V tile takes
// each token as 2- or 4-byte pieces, 8 tokens to a line, so a cache line of V is complete only
// once all the tokens of its half block are written: for a prompt those are consecutive tokens,
// and keeping them in one workgroup, with consecutive windows of a head on the same XCD
// (workgroup w runs on XCD w % 8; the logical window index is remapped so that each XCD owns a
// contiguous range), lets one L2 merge every line before it is written back.
template <int ESIZE>
__global__ void __launch_bounds__(256) append_kernel(uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
                                                     const uint8_t* __restrict__ key,
                                                     const uint8_t* __restrict__ value, int64_t key_stride_b,
                                                     int64_t value_stride_b, const int32_t* __restrict__ slots,
                                                     int32_t T, int32_t H, int32_t D, int32_t bs,
                                                     int32_t num_blocks, int32_t windows) {
  constexpr int EPC = 16 / ESIZE;  // elements per 16-byte chunk
  const int32_t chunks = D / EPC;
  const int32_t tw = 256 / chunks;  // tokens per window (chunks <= 256 is checked on the host)
  const int64_t per_xcd = gridDim.x / 8;  // the grid is a multiple of 8
  const int64_t logical = static_cast<int64_t>(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (logical >= static_cast<int64_t>(H) * windows || static_cast<int32_t>(threadIdx.x) >= tw * chunks) return;
  const int32_t h = static_cast<int32_t>(logical / windows);
  const int32_t c = static_cast<int32_t>(threadIdx.x) % chunks;
  const int64_t t = (logical % windows) * tw + static_cast<int32_t>(threadIdx.x) / chunks;
  if (t >= T) return;
  const int32_t slot = slots[t];
  if (slot < 0 || slot / bs >= num_blocks) return;  // -1 = skip; out-of-pool slots are never written
  const int64_t blk = slot / bs;
  const int32_t off = slot % bs;
  const int64_t src_off = static_cast<int64_t>(h) * D * ESIZE + static_cast<int64_t>(c) * 16;
  const u32x4 kv = *reinterpret_cast<const u32x4*>(key + t * key_stride_b + src_off);
  const u32x4 vv = *reinterpret_cast<const u32x4*>(value + t * value_stride_b + src_off);
  const int64_t head = blk * H + h;
  *reinterpret_cast<u32x4*>(k_cache + (head * bs * D) * ESIZE + static_cast<int64_t>(k_chunk_pos(off, c)) * 16) = kv;
  // Element (dimension d, token off) of the tile at ((off / 8) * D + d) * 8 + off % 8.
  uint8_t* vcol =
      v_cache + (head * D * bs + (static_cast<int64_t>(off >> 3) * D + static_cast<int64_t>(c) * EPC) * 8 + (off & 7)) *
                    ESIZE;
  if constexpr (ESIZE == 2) {
    const uint16_t* e = reinterpret_cast<const uint16_t*>(&vv);
#pragma unroll
    for (int i = 0; i < EPC; ++i) reinterpret_cast<uint16_t*>(vcol)[static_cast<int64_t>(i) * 8] = e[i];
  } else {
    const uint32_t* e = reinterpret_cast<const uint32_t*>(&vv);
#pragma unroll
    for (int i = 0; i < EPC; ++i) reinterpret_cast<uint32_t*>(vcol)[static_cast<int64_t>(i) * 8] = e[i];
  }
}

// grid.x = pair, grid.y = 0 for K / 1 for V; each workgroup copies one whole block of one tensor.
__global__ void __launch_bounds__(256) copy_blocks_kernel(uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
                                                          const int32_t* __restrict__ src_dst, int64_t block_bytes,
                                                          int32_t num_blocks) {
  const int32_t src = src_dst[2 * blockIdx.x];
  const int32_t dst = src_dst[2 * blockIdx.x + 1];
  if (src < 0 || dst < 0 || src >= num_blocks || dst >= num_blocks) return;  // out-of-pool pairs are skipped
  uint8_t* base = blockIdx.y == 0 ? k_cache : v_cache;
  const u32x4* s = reinterpret_cast<const u32x4*>(base + src * block_bytes);
  u32x4* d = reinterpret_cast<u32x4*>(base + dst * block_bytes);
  const int64_t n16 = block_bytes / 16;
  for (int64_t i = threadIdx.x; i < n16; i += blockDim.x) d[i] = s[i];
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int paged_cache_append(void* k_cache, void* v_cache, const void* key, const void* value,
                                  int64_t key_stride, int64_t value_stride, const int32_t* slot_mapping, int32_t T,
                                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                  int32_t dtype, pkv_stream_t stream) {
  if (!valid_dtype(dtype)) return fail(PKV_EINVAL, "paged_cache_append: unknown dtype %d", dtype);
  if (T < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail(PKV_EINVAL, "paged_cache_append: bad sizes T=%d Hkv=%d D=%d bs=%d N=%d", T, num_kv_heads, head_dim,
                block_size, num_blocks);
  const int es = elem_size(dtype);
  if (block_size != kBlock) return fail(PKV_EUNSUPPORTED, "paged_cache_append: block_size %d (16 only)", block_size);
  if ((static_cast<int64_t>(head_dim) * es) % 64 != 0)
    return fail(PKV_EUNSUPPORTED, "paged_cache_append: head_dim*elem_size must be a multiple of 64 bytes");
  if (T == 0) return PKV_OK;
  if (!k_cache || !v_cache || !key || !value || !slot_mapping)
    return fail(PKV_EINVAL, "paged_cache_append: NULL pointer");
  const int64_t row = static_cast<int64_t>(num_kv_heads) * head_dim;
  if (key_stride == 0) key_stride = row;
  if (value_stride == 0) value_stride = row;
  if (key_stride < row || value_stride < row)
    return fail(PKV_EINVAL, "paged_cache_append: token stride smaller than num_kv_heads*head_dim");
  if ((reinterpret_cast<uintptr_t>(key) | reinterpret_cast<uintptr_t>(value) | reinterpret_cast<uintptr_t>(k_cache) |
       reinterpret_cast<uintptr_t>(v_cache)) % 16 != 0 ||
      (key_stride * es) % 16 != 0 || (value_stride * es) % 16 != 0)
    return fail(PKV_EINVAL, "paged_cache_append: key/value/cache pointers and strides must be 16-byte aligned");
  const int chunks = head_dim * es / 16;
  if (chunks > 256) return fail(PKV_EUNSUPPORTED, "paged_cache_append: head_dim*elem_size above 4 KiB");
  const int tw = 256 / chunks;  // tokens per window
  const int64_t windows = (static_cast<int64_t>(T) + tw - 1) / tw;
  const int64_t grid = (static_cast<int64_t>(num_kv_heads) * windows + 7) / 8 * 8;
  if (grid > INT32_MAX || windows > INT32_MAX) return fail(PKV_EINVAL, "paged_cache_append: too many tokens");
  hipStream_t s = as_stream(stream);
  if (es == 2) {
    hipLaunchKernelGGL(append_kernel<2>, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, s,
                       static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache),
                       static_cast<const uint8_t*>(key), static_cast<const uint8_t*>(value), key_stride * es,
                       value_stride * es, slot_mapping, T, num_kv_heads, head_dim, block_size, num_blocks,
                       static_cast<int32_t>(windows));
  } else {
    hipLaunchKernelGGL(append_kernel<4>, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, s,
                       static_cast<uint8_t*>(k_cache), static_cast<uint8_t*>(v_cache),
                       static_cast<const uint8_t*>(key), static_cast<const uint8_t*>(value), key_stride * es,
                       value_stride * es, slot_mapping, T, num_kv_heads, head_dim, block_size, num_blocks,
                       static_cast<int32_t>(windows));
  }
  return check_launch("paged_cache_append");
}

extern "C" int paged_cache_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_dst, int32_t n,
                                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                       int32_t dtype, pkv_stream_t stream) {
  if (!valid_dtype(dtype)) return fail(PKV_EINVAL, "paged_cache_copy_blocks: unknown dtype %d", dtype);
  if (n < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail(PKV_EINVAL, "paged_cache_copy_blocks: bad sizes");
  if (n == 0) return PKV_OK;
  if (!k_cache || !v_cache || !src_dst) return fail(PKV_EINVAL, "paged_cache_copy_blocks: NULL pointer");
  const int64_t block_bytes = static_cast<int64_t>(num_kv_heads) * block_size * head_dim * elem_size(dtype);
  if (block_bytes % 16 != 0 ||
      (reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache)) % 16 != 0)
    return fail(PKV_EUNSUPPORTED, "paged_cache_copy_blocks: block size must be a multiple of 16 bytes, caches aligned");
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(n, 2), dim3(256), 0, as_stream(stream), static_cast<uint8_t*>(k_cache),
                     static_cast<uint8_t*>(v_cache), src_dst, block_bytes, num_blocks);
  return check_launch("paged_cache_copy_blocks");
}

extern "C" int paged_cache_copy_blocks_fp8(void* k_cache, void* v_cache, void* k_scale, void* v_scale,
                                           const int32_t* src_dst, int32_t n, int32_t num_kv_heads, int32_t head_dim,
                                           int32_t block_size, int32_t num_blocks, pkv_stream_t stream) {
  if (n < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail(PKV_EINVAL, "paged_cache_copy_blocks_fp8: bad sizes");
  if (n == 0) return PKV_OK;
  if (!k_cache || !v_cache || !k_scale || !v_scale || !src_dst)
    return fail(PKV_EINVAL, "paged_cache_copy_blocks_fp8: NULL pointer");
  const int64_t code_bytes = static_cast<int64_t>(num_kv_heads) * block_size * head_dim;
  const int64_t scale_bytes = static_cast<int64_t>(num_kv_heads) * block_size * 4;
  if (code_bytes % 16 != 0 || scale_bytes % 16 != 0 ||
      (reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache) |
       reinterpret_cast<uintptr_t>(k_scale) | reinterpret_cast<uintptr_t>(v_scale)) % 16 != 0)
    return fail(PKV_EUNSUPPORTED, "paged_cache_copy_blocks_fp8: blocks must be multiples of 16 bytes, arrays aligned");
  hipStream_t s = as_stream(stream);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(n, 2), dim3(256), 0, s, static_cast<uint8_t*>(k_cache),
                     static_cast<uint8_t*>(v_cache), src_dst, code_bytes, num_blocks);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(n, 2), dim3(64), 0, s, static_cast<uint8_t*>(k_scale),
                     static_cast<uint8_t*>(v_scale), src_dst, scale_bytes, num_blocks);
  return check_launch("paged_cache_copy_blocks_fp8");
}
