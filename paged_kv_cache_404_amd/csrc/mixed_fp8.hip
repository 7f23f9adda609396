// One launch for a continuous-batching step's attention over the FP8 (E4M3) cache: the decode
// rows of a batch and the rows of up to 16 prefill chunks.
//
// The step is the one csrc/mixed.hip runs over bf16 / fp16 caches ([Chapter] "Continuous
// batching and PagedAttention", "How the scheduler works", and [Notes] "Continuous batching and
// PagedAttention: serving many users from one GPU", "Prefill gets in the way": the running
// sequences' decode tokens and a chunk of a new prompt in one batch), over the quantised cache
// ([Notes] "Memory, not compute, caps the batch").  Workgroups [0, n_dec) each run one (KV head,
// sequence, partition) of the FP8 decode (decode_fp8_part.h), the rest one (16-row tile, KV head)
// of a chunk (prefill_tile with FP8 set).  Every output is bit for bit the one
// paged_attention_decode_fp8 / paged_attention_prefill_chunk_fp8 produce; with split-K
// partitions the decode's log-sum-exp merge follows as a second launch.
#include <cmath>

#include "decode_fp8_part.h"
#include "mixed_host.h"

namespace pkv {
namespace {

struct MixedFp8Args {
  Fp8Args dec;
  int32_t B_dec;
  int32_t n_dec_wg;  // Hkv * B_dec * max_parts rounded up to a multiple of 8
  ChunkSet pre;
};

// NWD: decode waves (4 or 8, the FP8 decode's rule for the partition size).  Every workgroup has
// 8 waves; a 4-wave decode workgroup's other 4 waves leave at once (a barrier then waits for the
// remaining waves only).
template <int DT, int DT_OUT, int D, int G, int NWD>
__global__ void __launch_bounds__(512) mixed_fp8_kernel(MixedFp8Args m) {
  static_assert(PrefillShape<G>::NWAVES == 8, "the mixed launch runs 8-wave prefill tiles");
  constexpr int kDec = fp8_decode_smem_floats<D, G, NWD>();
  constexpr int kPre = prefill_smem_floats<D, G>();
  __shared__ float smem[smax(kDec, kPre)];
  const int id = blockIdx.x;
  if (id < m.n_dec_wg) {
    const int g = id % m.pre.Hkv;
    const int y = (id / m.pre.Hkv) % m.B_dec;
    const int z = id / (m.pre.Hkv * m.B_dec);
    if (z >= m.dec.max_parts) return;  // padding up to a multiple of 8
    if (NWD < 8 && threadIdx.x >= NWD * 64) return;
    decode_fp8_part<DT, DT_OUT, D, G, NWD, false>(m.dec, g, y, z, smem);
    return;
  }
  mixed_prefill_role<DT, DT_OUT, D, G, true>(m.pre, id, smem);
}

template <int DT, int DT_OUT, int D, int G>
void launch_fp8_nw(const MixedFp8Args& m, bool wide, int grid, hipStream_t s) {
  if (wide)
    hipLaunchKernelGGL((mixed_fp8_kernel<DT, DT_OUT, D, G, 8>), dim3(grid), dim3(512), 0, s, m);
  else
    hipLaunchKernelGGL((mixed_fp8_kernel<DT, DT_OUT, D, G, 4>), dim3(grid), dim3(512), 0, s, m);
}

template <int DT, int DT_OUT, int D>
void launch_fp8_g(const MixedFp8Args& m, bool wide, int grid, hipStream_t s) {
  switch (m.pre.Hq / m.pre.Hkv) {
    case 1: launch_fp8_nw<DT, DT_OUT, D, 1>(m, wide, grid, s); break;
    case 2: launch_fp8_nw<DT, DT_OUT, D, 2>(m, wide, grid, s); break;
    case 4: launch_fp8_nw<DT, DT_OUT, D, 4>(m, wide, grid, s); break;
    default: launch_fp8_nw<DT, DT_OUT, D, 8>(m, wide, grid, s); break;
  }
}

template <int DT, int DT_OUT>
void launch_fp8_d(const MixedFp8Args& m, int D, bool wide, int grid, hipStream_t s) {
  if (D == 64)
    launch_fp8_g<DT, DT_OUT, 64>(m, wide, grid, s);
  else
    launch_fp8_g<DT, DT_OUT, 128>(m, wide, grid, s);
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int paged_attention_mixed_fp8(void* dec_out, const void* dec_query, const int32_t* dec_block_tables,
                                         const int32_t* dec_context_lens, int32_t B_dec, int32_t dec_max_blocks,
                                         int32_t dec_max_context_len, const int32_t* host_dec_context_lens,
                                         int32_t dec_partition_size, void* workspace, size_t workspace_bytes,
                                         void* pre_out, const void* pre_query, const int32_t* pre_block_tables,
                                         int32_t pre_max_blocks, const int32_t* host_ctx_starts,
                                         const int32_t* host_chunk_lens, int32_t num_chunks, int32_t out_dtype,
                                         const void* k_cache, const void* v_cache, const void* k_scale,
                                         const void* v_scale, int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                                         int32_t q_dtype, pkv_stream_t stream) {
  const char* fn = "paged_attention_mixed_fp8";
  if (q_dtype != PKV_BF16 && q_dtype != PKV_F16)
    return fail(PKV_EUNSUPPORTED, "%s: query dtype %d (bf16 or fp16)", fn, q_dtype);
  if (out_dtype != PKV_F32 && out_dtype != q_dtype)
    return fail(PKV_EINVAL, "%s: out_dtype must be PKV_F32 or the query dtype", fn);
  if (B_dec < 0 || num_chunks < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 || block_size <= 0 ||
      dec_max_blocks < 0 || pre_max_blocks < 0 || dec_max_context_len < 0)
    return fail(PKV_EINVAL, "%s: bad sizes", fn);
  if (num_q_heads % num_kv_heads != 0) return fail(PKV_EINVAL, "%s: num_q_heads not a multiple of num_kv_heads", fn);
  // The prefill tile compares raw scores against thresholds divided by the scale: positive only.
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(PKV_EINVAL, "%s: scale must be positive and finite", fn);
  const int G = num_q_heads / num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(PKV_EUNSUPPORTED, "%s: group size %d", fn, G);
  if (block_size != kBlock) return fail(PKV_EUNSUPPORTED, "%s: block_size %d (kernels implement 16)", fn, block_size);
  if (head_dim != 64 && head_dim != 128) return fail(PKV_EUNSUPPORTED, "%s: head_dim %d", fn, head_dim);
  if (num_chunks > kMaxChunks) return fail(PKV_EUNSUPPORTED, "%s: more than %d prefill chunks", fn, kMaxChunks);
  if (!k_cache || !v_cache || !k_scale || !v_scale) return fail(PKV_EINVAL, "%s: NULL cache or scales", fn);
  if (num_chunks > 0 && (!pre_out || !pre_query || !pre_block_tables || !host_ctx_starts || !host_chunk_lens))
    return fail(PKV_EINVAL, "%s: NULL prefill pointer", fn);
  if ((reinterpret_cast<uintptr_t>(pre_query) | reinterpret_cast<uintptr_t>(k_cache) |
       reinterpret_cast<uintptr_t>(v_cache) | reinterpret_cast<uintptr_t>(k_scale) |
       reinterpret_cast<uintptr_t>(v_scale)) % 16 != 0)
    return fail(PKV_EINVAL, "%s: queries, caches and scales must be 16-byte aligned", fn);
  MixedFp8Args m{};
  // The decode part: paged_attention_decode_fp8's argument rules, partition plan and work order.
  bool wide = true, empty = true;
  if (B_dec > 0) {
    const int st = fp8_setup(fn, m.dec, wide, empty, dec_out, out_dtype, dec_query, k_cache, v_cache, k_scale,
                             v_scale, dec_block_tables, dec_context_lens, B_dec, num_q_heads, num_kv_heads,
                             head_dim, block_size, dec_max_blocks, num_blocks, dec_max_context_len, scale,
                             dec_partition_size, workspace, workspace_bytes, q_dtype, host_dec_context_lens, nullptr,
                             nullptr);
    if (st != PKV_OK) return st;
  }
  const bool has_dec = !empty;
  m.B_dec = has_dec ? B_dec : 1;
  if (!has_dec) m.dec.max_parts = 0;
  int64_t wg = has_dec ? (static_cast<int64_t>(num_kv_heads) * B_dec * m.dec.max_parts + 7) / 8 * 8 : 0;
  m.n_dec_wg = static_cast<int32_t>(wg);
  m.pre.k = k_cache;
  m.pre.v = v_cache;
  m.pre.ksc = static_cast<const float*>(k_scale);
  m.pre.vsc = static_cast<const float*>(v_scale);
  m.pre.Hq = num_q_heads;
  m.pre.Hkv = num_kv_heads;
  m.pre.num_blocks = num_blocks;
  m.pre.scale_log2 = scale * kLog2e;
  // prefill chunks, rows packed one after another in pre_query / pre_out
  const int pst = pack_chunks(fn, m.pre, wg, pre_out, pre_query, pre_block_tables, pre_max_blocks, host_ctx_starts,
                              host_chunk_lens, num_chunks, head_dim, elem_size(q_dtype), elem_size(out_dtype));
  if (pst != PKV_OK) return pst;
  if (wg == 0) return PKV_OK;
  hipStream_t s = as_stream(stream);
  const bool f32out = out_dtype == PKV_F32;
  const int grid = static_cast<int>(wg);
  if (q_dtype == PKV_BF16) {
    if (f32out)
      launch_fp8_d<PKV_BF16, PKV_F32>(m, head_dim, wide, grid, s);
    else
      launch_fp8_d<PKV_BF16, PKV_BF16>(m, head_dim, wide, grid, s);
  } else {
    if (f32out)
      launch_fp8_d<PKV_F16, PKV_F32>(m, head_dim, wide, grid, s);
    else
      launch_fp8_d<PKV_F16, PKV_F16>(m, head_dim, wide, grid, s);
  }
  const int st = check_launch(fn);
  if (st != PKV_OK || !has_dec || m.dec.max_parts <= 1) return st;
  return paged_attention_decode_reduce(dec_out, out_dtype, dec_context_lens, B_dec, num_q_heads, head_dim,
                                       dec_max_context_len, dec_partition_size, workspace, workspace_bytes, stream);
}
