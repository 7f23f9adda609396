// Chunked-prefill causal attention against the FP8 (E4M3) cache.
//
// What is computed is the prefill of csrc/prefill.hip ([Chapter] "How the scheduler works",
// [Notes] "Prefill gets in the way": row i of a chunk sits at position ctx_start + i and attends
// to positions 0 .. ctx_start + i), over the values the quantised cache stands for (code times its
// slot's scale; [Notes] "Memory, not compute, caps the batch" is why the cache is quantised).
// The workgroup tiling is the bf16 one (prefill_tile with FP8 set): codes are widened exactly to
// the query's type in registers for the same v_mfma_f32_16x16x32 products, and the per-slot K
// and V scales multiply scores and weights outside the products.
#include <cmath>

#include "prefill_tile.h"

namespace pkv {
namespace {

template <int DT, int DT_OUT, int D, int G>
__global__ void __launch_bounds__(PrefillShape<G>::NWAVES * 64) prefill_fp8_kernel(PrefillArgs a) {
  __shared__ float smem[prefill_smem_floats<D, G>()];
  prefill_tile<DT, DT_OUT, D, G, true>(a, blockIdx.x, smem);
}

template <int DT, int DT_OUT, int D>
void launch_fp8_g(const PrefillArgs& a, hipStream_t s) {
  const dim3 grid(a.row_tiles * a.Hkv);
  switch (a.Hq / a.Hkv) {
    case 1: hipLaunchKernelGGL((prefill_fp8_kernel<DT, DT_OUT, D, 1>), grid, dim3(PrefillShape<1>::NWAVES * 64), 0, s, a); break;
    case 2: hipLaunchKernelGGL((prefill_fp8_kernel<DT, DT_OUT, D, 2>), grid, dim3(PrefillShape<2>::NWAVES * 64), 0, s, a); break;
    case 4: hipLaunchKernelGGL((prefill_fp8_kernel<DT, DT_OUT, D, 4>), grid, dim3(PrefillShape<4>::NWAVES * 64), 0, s, a); break;
    default: hipLaunchKernelGGL((prefill_fp8_kernel<DT, DT_OUT, D, 8>), grid, dim3(PrefillShape<8>::NWAVES * 64), 0, s, a); break;
  }
}

template <int DT, int DT_OUT>
void launch_fp8_d(const PrefillArgs& a, int D, hipStream_t s) {
  if (D == 64)
    launch_fp8_g<DT, DT_OUT, 64>(a, s);
  else
    launch_fp8_g<DT, DT_OUT, 128>(a, s);
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int paged_attention_prefill_chunk_fp8(void* out, int32_t out_dtype, const void* query, const void* k_cache,
                                                 const void* v_cache, const void* k_scale, const void* v_scale,
                                                 const int32_t* block_table, int32_t ctx_start, int32_t C,
                                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                                 int32_t block_size, int32_t num_blocks, float scale, int32_t q_dtype,
                                                 pkv_stream_t stream) {
  const char* fn = "paged_attention_prefill_chunk_fp8";
  if (q_dtype != PKV_BF16 && q_dtype != PKV_F16)
    return fail(PKV_EUNSUPPORTED, "%s: query dtype %d (bf16 or fp16)", fn, q_dtype);
  if (out_dtype != PKV_F32 && out_dtype != q_dtype)
    return fail(PKV_EINVAL, "%s: out_dtype must be PKV_F32 or the query dtype", fn);
  if (ctx_start < 0 || C < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 || block_size <= 0)
    return fail(PKV_EINVAL, "%s: bad sizes", fn);
  if (num_q_heads % num_kv_heads != 0) return fail(PKV_EINVAL, "%s: num_q_heads not a multiple of num_kv_heads", fn);
  // The tile compares raw scores against thresholds divided by the scale: positive only.
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(PKV_EINVAL, "%s: scale must be positive and finite", fn);
  if (block_size != kBlock) return fail(PKV_EUNSUPPORTED, "%s: block_size %d (kernels implement 16)", fn, block_size);
  if (head_dim != 64 && head_dim != 128) return fail(PKV_EUNSUPPORTED, "%s: head_dim %d (64 or 128)", fn, head_dim);
  const int G = num_q_heads / num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(PKV_EUNSUPPORTED, "%s: group size %d", fn, G);
  if (static_cast<int64_t>(ctx_start) + C > static_cast<int64_t>(num_blocks) * block_size)
    return fail(PKV_EINVAL, "%s: ctx_start + C exceeds the pool", fn);
  if (C == 0) return PKV_OK;
  if (!out || !query || !k_cache || !v_cache || !k_scale || !v_scale || !block_table)
    return fail(PKV_EINVAL, "%s: NULL pointer", fn);
  if ((reinterpret_cast<uintptr_t>(query) | reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache) |
       reinterpret_cast<uintptr_t>(k_scale) | reinterpret_cast<uintptr_t>(v_scale)) % 16 != 0)
    return fail(PKV_EINVAL, "%s: query, caches and scales must be 16-byte aligned", fn);
  const int64_t tiles = (static_cast<int64_t>(C) + 15) / 16;
  if (tiles * num_kv_heads > INT32_MAX) return fail(PKV_EINVAL, "%s: chunk too large", fn);
  PrefillArgs a{};
  a.out = out;
  a.q = query;
  a.k = k_cache;
  a.v = v_cache;
  a.ksc = static_cast<const float*>(k_scale);
  a.vsc = static_cast<const float*>(v_scale);
  a.table = block_table;
  a.ctx_start = ctx_start;
  a.C = C;
  a.Hq = num_q_heads;
  a.Hkv = num_kv_heads;
  a.num_blocks = num_blocks;
  a.row_tiles = static_cast<int32_t>(tiles);
  a.scale_log2 = scale * kLog2e;
  hipStream_t s = as_stream(stream);
  const bool f32out = out_dtype == PKV_F32;
  if (q_dtype == PKV_BF16) {
    if (f32out)
      launch_fp8_d<PKV_BF16, PKV_F32>(a, head_dim, s);
    else
      launch_fp8_d<PKV_BF16, PKV_BF16>(a, head_dim, s);
  } else {
    if (f32out)
      launch_fp8_d<PKV_F16, PKV_F32>(a, head_dim, s);
    else
      launch_fp8_d<PKV_F16, PKV_F16>(a, head_dim, s);
  }
  return check_launch(fn);
}
