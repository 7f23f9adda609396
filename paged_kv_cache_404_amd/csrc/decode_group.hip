// Grouped paged decode: sequences that share cached blocks (forked samples, common prefixes) run
// group_size to a workgroup, and a step whose blocks are common to the group is read once for all
// of them.  The body and its guarantees are described at the top of csrc/decode_group.h: every
// output is bit for bit that of paged_attention_decode with the same partition_size.
#include "decode_group.h"
#include "decode_host.h"

namespace pkv {
namespace {

// At least two waves per SIMD whatever NW (the 4-wave workgroups would otherwise take up to 512
// registers per lane and run one wave per SIMD).
template <int DT, int DT_OUT, int D, int G, int NS, int NW>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
decode_group_kernel(DecodeArgs a, int32_t B) {
  __shared__ float smem[group_smem_floats<D, G, NS, NW>()];
  decode_group_part<DT, DT_OUT, D, G, NS, NW>(a, B, blockIdx.x, blockIdx.y, blockIdx.z, smem);
}

template <int DT, int DT_OUT, int D, int G, int NS>
void launch_ns(const DecodeArgs& a, int B, int ngroups, int nw, hipStream_t s) {
  const dim3 grid(a.Hkv, ngroups, a.max_parts);
  if (nw == 4)
    hipLaunchKernelGGL((decode_group_kernel<DT, DT_OUT, D, G, NS, 4>), grid, dim3(256), 0, s, a, B);
  else
    hipLaunchKernelGGL((decode_group_kernel<DT, DT_OUT, D, G, NS, 8>), grid, dim3(512), 0, s, a, B);
}

// Group sizes whose columns (group_size x query heads per KV head) fill 8 or 16 matrix columns.
template <int DT, int DT_OUT, int D>
bool launch_gs(const DecodeArgs& a, int B, int G, int NS, int ngroups, int nw, hipStream_t s) {
  switch (G * 100 + NS) {
    case 108: launch_ns<DT, DT_OUT, D, 1, 8>(a, B, ngroups, nw, s); return true;
    case 116: launch_ns<DT, DT_OUT, D, 1, 16>(a, B, ngroups, nw, s); return true;
    case 204: launch_ns<DT, DT_OUT, D, 2, 4>(a, B, ngroups, nw, s); return true;
    case 208: launch_ns<DT, DT_OUT, D, 2, 8>(a, B, ngroups, nw, s); return true;
    case 402: launch_ns<DT, DT_OUT, D, 4, 2>(a, B, ngroups, nw, s); return true;
    case 404: launch_ns<DT, DT_OUT, D, 4, 4>(a, B, ngroups, nw, s); return true;
    case 802: launch_ns<DT, DT_OUT, D, 8, 2>(a, B, ngroups, nw, s); return true;
    default: return false;
  }
}

template <int DT, int DT_OUT>
bool launch_dim(const DecodeArgs& a, int B, int D, int G, int NS, int ngroups, int nw, hipStream_t s) {
  return D == 64 ? launch_gs<DT, DT_OUT, 64>(a, B, G, NS, ngroups, nw, s)
                 : launch_gs<DT, DT_OUT, 128>(a, B, G, NS, ngroups, nw, s);
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int paged_attention_decode_grouped(void* out, int32_t out_dtype, const void* query, const void* k_cache,
                                              const void* v_cache, const int32_t* block_tables,
                                              const int32_t* context_lens, int32_t B, int32_t num_q_heads,
                                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                              int32_t max_blocks_per_seq, int32_t num_blocks,
                                              int32_t max_context_len, float scale, int32_t partition_size,
                                              void* workspace, size_t workspace_bytes, int32_t dtype,
                                              int32_t group_size, pkv_stream_t stream) {
  const char* fn = "paged_attention_decode_grouped";
  int st = validate(fn, out, out_dtype, query, k_cache, v_cache, block_tables, context_lens, B, num_q_heads,
                    num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, max_context_len,
                    partition_size, workspace, workspace_bytes, dtype);
  if (st != PKV_OK) return st;
  const int G = num_q_heads / num_kv_heads;
  if (group_size < 1) return fail(PKV_EINVAL, "%s: group_size %d", fn, group_size);
  if (group_size == 1)
    return paged_attention_decode(out, out_dtype, query, k_cache, v_cache, block_tables, context_lens, B, num_q_heads,
                                  num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                                  max_context_len, scale, partition_size, workspace, workspace_bytes, dtype, nullptr,
                                  stream);
  if (dtype == PKV_F32) return fail(PKV_EUNSUPPORTED, "%s: groups need bf16 or fp16 caches", fn);
  const int cols = group_size * G;
  if (cols != 8 && cols != 16)
    return fail(PKV_EUNSUPPORTED, "%s: group_size x (num_q_heads / num_kv_heads) = %d, must be 8 or 16", fn, cols);
  if (B == 0 || max_context_len == 0) return PKV_OK;
  const Plan pl = make_plan(B, num_q_heads, head_dim, max_context_len, partition_size);
  DecodeArgs a{};
  a.out = out;
  a.q = query;
  a.k = k_cache;
  a.v = v_cache;
  a.tables = block_tables;
  a.lens = context_lens;
  a.part_ml = pl.need_bytes ? static_cast<float*>(workspace) : nullptr;
  a.part_o = pl.need_bytes ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + pl.ml_bytes) : nullptr;
  a.Hq = num_q_heads;
  a.Hkv = num_kv_heads;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.max_parts = pl.max_parts;
  a.part_size = pl.part_size;
  a.scale_log2 = scale * kLog2e;
  const int ngroups = (B + group_size - 1) / group_size;
  const int nw = decode_waves(partition_size, pl);
  hipStream_t s = as_stream(stream);
  const bool f32out = out_dtype == PKV_F32;
  bool ok;
  if (dtype == PKV_BF16)
    ok = f32out ? launch_dim<PKV_BF16, PKV_F32>(a, B, head_dim, G, group_size, ngroups, nw, s)
                : launch_dim<PKV_BF16, PKV_BF16>(a, B, head_dim, G, group_size, ngroups, nw, s);
  else
    ok = f32out ? launch_dim<PKV_F16, PKV_F32>(a, B, head_dim, G, group_size, ngroups, nw, s)
                : launch_dim<PKV_F16, PKV_F16>(a, B, head_dim, G, group_size, ngroups, nw, s);
  if (!ok) return fail(PKV_EUNSUPPORTED, "%s: group_size %d with group %d", fn, group_size, G);
  st = check_launch(fn);
  if (st != PKV_OK) return st;
  return paged_attention_decode_reduce(out, out_dtype, context_lens, B, num_q_heads, head_dim, max_context_len,
                                       partition_size, workspace, workspace_bytes, stream);
}
