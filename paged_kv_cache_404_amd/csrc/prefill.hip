// Chunked-prefill causal attention against the paged cache.
//
// [Chapter] "Continuous batching and PagedAttention", "How the scheduler works", and [Notes]
// "Continuous batching and PagedAttention: serving many users from one GPU", "Prefill gets in
// the way": a long prompt is prefilled in chunks that fit the step's token budget and are
// interleaved with decode steps.  Row i of a chunk sits at absolute position ctx_start + i, its
// K/V are already in the cache, and it attends causally to positions 0 .. ctx_start + i through
// the sequence's block table.  Per row the arithmetic is the decode's (scaled dot products,
// softmax, weighted sum of values; [Serving] "Production Serving: Continuous Batching and
// PagedAttention", The Build, Step 6).
//
// MI355X mapping (bf16 / fp16; fp32 caches take a plain vector-ALU kernel): a workgroup owns 16
// consecutive chunk rows of the G query heads of one KV
// head; its waves split the key range and the heads, and each wave serves two heads from every
// K/V fragment it loads.  Per
// 32-key step, S^T = K.Q^T (2 x D/32 MFMA 16x16x32) and O += P.V (D/16 MFMA, twice: P split
// into hi + lo 16-bit rows so the weights keep ~16 mantissa bits).  The causal limit only masks
// the last steps of each row tile.  Workgroups are ordered so that consecutive ids on one XCD
// work on the same KV head (its K/V then stay in that XCD's L2).
#include <cmath>

#include "prefill_tile.h"
#include "prefill_valu.h"

namespace pkv {
namespace {

template <int DT, int DT_OUT, int D, int G>
__global__ void __launch_bounds__(PrefillShape<G>::NWAVES * 64) prefill_mfma_kernel(PrefillArgs a) {
  __shared__ float smem[prefill_smem_floats<D, G>()];
  prefill_tile<DT, DT_OUT, D, G>(a, blockIdx.x, smem);
}

// grid = (Hq, C): one wave per (query head, chunk row).
template <int DT_OUT, int D>
__global__ void __launch_bounds__(64) prefill_valu_kernel(PrefillArgs a) {
  prefill_valu_part<DT_OUT, D>(a, blockIdx.x, blockIdx.y);
}

template <int DT, int DT_OUT, int D, int G>
void launch_one(const PrefillArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((prefill_mfma_kernel<DT, DT_OUT, D, G>), dim3(a.row_tiles * a.Hkv),
                     dim3(PrefillShape<G>::NWAVES * 64), 0, s, a);
}

template <int DT, int DT_OUT, int D>
void launch_g(const PrefillArgs& a, hipStream_t s) {
  switch (a.Hq / a.Hkv) {
    case 1: launch_one<DT, DT_OUT, D, 1>(a, s); break;
    case 2: launch_one<DT, DT_OUT, D, 2>(a, s); break;
    case 4: launch_one<DT, DT_OUT, D, 4>(a, s); break;
    default: launch_one<DT, DT_OUT, D, 8>(a, s); break;
  }
}

template <int DT, int DT_OUT>
void launch_d(const PrefillArgs& a, int D, hipStream_t s) {
  if (D == 64)
    launch_g<DT, DT_OUT, 64>(a, s);
  else
    launch_g<DT, DT_OUT, 128>(a, s);
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int paged_attention_prefill_chunk(void* out, int32_t out_dtype, const void* query, const void* k_cache,
                                             const void* v_cache, const int32_t* block_table, int32_t ctx_start,
                                             int32_t C, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                             int32_t block_size, int32_t num_blocks, float scale, int32_t dtype,
                                             pkv_stream_t stream) {
  const char* fn = "paged_attention_prefill_chunk";
  if (!valid_dtype(dtype)) return fail(PKV_EINVAL, "%s: unknown dtype %d", fn, dtype);
  if (out_dtype != PKV_F32 && out_dtype != dtype)
    return fail(PKV_EINVAL, "%s: out_dtype must be PKV_F32 or the input dtype", fn);
  if (ctx_start < 0 || C < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 || block_size <= 0)
    return fail(PKV_EINVAL, "%s: bad sizes", fn);
  if (num_q_heads % num_kv_heads != 0) return fail(PKV_EINVAL, "%s: num_q_heads not a multiple of num_kv_heads", fn);
  // The prefill tile compares raw scores against thresholds divided by the scale: positive only.
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(PKV_EINVAL, "%s: scale must be positive and finite", fn);
  if (block_size != kBlock) return fail(PKV_EUNSUPPORTED, "%s: block_size %d (kernels implement 16)", fn, block_size);
  if (head_dim != 64 && head_dim != 128) return fail(PKV_EUNSUPPORTED, "%s: head_dim %d", fn, head_dim);
  const int G = num_q_heads / num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(PKV_EUNSUPPORTED, "%s: group size %d", fn, G);
  if (static_cast<int64_t>(ctx_start) + C > static_cast<int64_t>(num_blocks) * block_size)
    return fail(PKV_EINVAL, "%s: ctx_start + C exceeds the pool", fn);
  if (C == 0) return PKV_OK;
  if (!out || !query || !k_cache || !v_cache || !block_table) return fail(PKV_EINVAL, "%s: NULL pointer", fn);
  if ((reinterpret_cast<uintptr_t>(query) | reinterpret_cast<uintptr_t>(k_cache) |
       reinterpret_cast<uintptr_t>(v_cache)) % 16 != 0)
    return fail(PKV_EINVAL, "%s: query and caches must be 16-byte aligned", fn);
  const int64_t tiles = (static_cast<int64_t>(C) + 15) / 16;
  if (tiles * num_kv_heads > INT32_MAX) return fail(PKV_EINVAL, "%s: chunk too large", fn);
  if (dtype == PKV_F32 && C > 65535) return fail(PKV_EUNSUPPORTED, "%s: fp32 chunks of more than 65535 rows", fn);
  PrefillArgs a{};
  a.out = out;
  a.q = query;
  a.k = k_cache;
  a.v = v_cache;
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
  if (dtype == PKV_F32) {
    const dim3 grid(num_q_heads, C);
    if (head_dim == 64)
      hipLaunchKernelGGL((prefill_valu_kernel<PKV_F32, 64>), grid, dim3(64), 0, s, a);
    else
      hipLaunchKernelGGL((prefill_valu_kernel<PKV_F32, 128>), grid, dim3(64), 0, s, a);
  } else if (dtype == PKV_BF16) {
    if (f32out)
      launch_d<PKV_BF16, PKV_F32>(a, head_dim, s);
    else
      launch_d<PKV_BF16, PKV_BF16>(a, head_dim, s);
  } else {
    if (f32out)
      launch_d<PKV_F16, PKV_F32>(a, head_dim, s);
    else
      launch_d<PKV_F16, PKV_F16>(a, head_dim, s);
  }
  return check_launch(fn);
}
