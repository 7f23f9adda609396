// One launch for a whole continuous-batching step's attention: the decode rows of a batch and the
// rows of any number of prefill chunks.
//
// [Chapter] "Continuous batching and PagedAttention", "How the scheduler works", and [Notes]
// "Continuous batching and PagedAttention: serving many users from one GPU", "Prefill gets in the
// way": a step carries the running sequences' decode tokens and, within the token budget, a chunk
// of a new prompt; production servers put both into the same batch.  Here they go into the same
// kernel launch: workgroups [0, n_dec) each run one (KV head, sequence or group of sequences,
// partition) of the decode (the body of the decode kernel, or of the grouped decode kernel when
// sequences share blocks), the rest each run one (16-row tile, KV head) of a prefill chunk (the
// body of the prefill kernel).  Decode work is dispatched first: its workgroups stream the cache
// from HBM while the prefill workgroups, which are bound by the matrix and vector units, fill the
// other compute units.  With split-K partitions the decode's log-sum-exp merge follows as a second
// launch.  Every output is bit for bit the one the separate launches produce (same bodies, same
// order of arithmetic).  LDS is one buffer, used by whichever body the workgroup runs.
#include <algorithm>
#include <cmath>

#include "decode_group.h"
#include "decode_host.h"
#include "decode_valu.h"
#include "mixed_host.h"
#include "prefill_valu.h"

namespace pkv {
namespace {

struct MixedArgs {
  DecodeArgs dec;
  int32_t B_dec;
  int32_t dec_rows;  // decode rows of the grid: B_dec sequences, or ceil(B_dec / NS) groups
  int32_t n_dec_wg;  // Hkv * dec_rows * max_parts rounded up to a multiple of 8
  ChunkSet pre;
};

// NS: decode sequences per workgroup (1, or a grouped size); NWD: decode waves (4 or 8, the
// decode kernel's rule for the partition size).  Every workgroup has 8 waves; a 4-wave decode
// workgroup's other 4 waves leave at once (a barrier then waits for the remaining waves only).
template <int DT, int DT_OUT, int D, int G, int NS, int NWD>
__global__ void __launch_bounds__(512) mixed_kernel(MixedArgs m) {
  static_assert(PrefillShape<G>::NWAVES == 8, "the mixed launch runs 8-wave prefill tiles");
  constexpr int kDec = NS == 1 ? decode_smem_floats<D, G, NWD>() : group_smem_floats<D, G, NS, NWD>();
  constexpr int kPre = prefill_smem_floats<D, G>();
  __shared__ float smem[smax(kDec, kPre)];
  const int id = blockIdx.x;
  if (id < m.n_dec_wg) {
    const int g = id % m.pre.Hkv;
    const int y = (id / m.pre.Hkv) % m.dec_rows;
    const int z = id / (m.pre.Hkv * m.dec_rows);
    if (z >= m.dec.max_parts) return;  // padding up to a multiple of 8
    if (NWD < 8 && threadIdx.x >= NWD * 64) return;
    if constexpr (NS == 1)
      decode_mfma_part<DT, DT_OUT, D, G, NWD, false>(m.dec, g, y, z, smem);
    else
      decode_group_part<DT, DT_OUT, D, G, NS, NWD>(m.dec, m.B_dec, g, y, z, smem);
    return;
  }
  mixed_prefill_role<DT, DT_OUT, D, G, false>(m.pre, id, smem);
}

template <int DT, int DT_OUT, int D, int G, int NS>
void launch_nw(const MixedArgs& m, int nwd, int grid, hipStream_t s) {
  if (nwd == 4)
    hipLaunchKernelGGL((mixed_kernel<DT, DT_OUT, D, G, NS, 4>), dim3(grid), dim3(512), 0, s, m);
  else
    hipLaunchKernelGGL((mixed_kernel<DT, DT_OUT, D, G, NS, 8>), dim3(grid), dim3(512), 0, s, m);
}

// Decode grouping: 1, or mixed_group_size(G) sequences per workgroup.
constexpr int mixed_group_size(int G) { return G >= 4 ? 2 : 8 / G; }

template <int DT, int DT_OUT, int D, int G>
void launch_ns(const MixedArgs& m, int ns, int nwd, int grid, hipStream_t s) {
  constexpr int kGroup = mixed_group_size(G);
  if (ns == 1)
    launch_nw<DT, DT_OUT, D, G, 1>(m, nwd, grid, s);
  else
    launch_nw<DT, DT_OUT, D, G, kGroup>(m, nwd, grid, s);
}

template <int DT, int DT_OUT, int D>
void launch_g(const MixedArgs& m, int ns, int nwd, int grid, hipStream_t s) {
  switch (m.pre.Hq / m.pre.Hkv) {
    case 1: launch_ns<DT, DT_OUT, D, 1>(m, ns, nwd, grid, s); break;
    case 2: launch_ns<DT, DT_OUT, D, 2>(m, ns, nwd, grid, s); break;
    case 4: launch_ns<DT, DT_OUT, D, 4>(m, ns, nwd, grid, s); break;
    default: launch_ns<DT, DT_OUT, D, 8>(m, ns, nwd, grid, s); break;
  }
}

template <int DT, int DT_OUT>
void launch_d(const MixedArgs& m, int D, int ns, int nwd, int grid, hipStream_t s) {
  if (D == 64)
    launch_g<DT, DT_OUT, 64>(m, ns, nwd, grid, s);
  else
    launch_g<DT, DT_OUT, 128>(m, ns, nwd, grid, s);
}

// fp32 caches: the vector-ALU bodies, one wave per workgroup.  Workgroups [0, n_dec_wg) run a
// (query head, sequence, partition) of the decode (decode_valu_part, the fp32 decode kernel's
// body), the rest a (query head, row) of a chunk (prefill_valu_part, the fp32 prefill kernel's).
struct MixedValuArgs {
  DecodeArgs dec;
  int32_t B_dec;
  int32_t n_dec_wg;  // Hq * B_dec * max_parts
  ChunkSet pre;      // chunk i runs Hq * C workgroups from chunks[i].wg_base on
};

template <int DT_OUT, int D>
__global__ void __launch_bounds__(64) mixed_valu_kernel(MixedValuArgs m) {
  const int id = blockIdx.x;
  if (id < m.n_dec_wg) {
    const int hq = id % m.dec.Hq;
    const int y = (id / m.dec.Hq) % m.B_dec;
    const int z = id / (m.dec.Hq * m.B_dec);
    decode_valu_part<PKV_F32, DT_OUT, D>(m.dec, hq, y, z);
    return;
  }
  int c = 0;
  while (c + 1 < m.pre.n_chunks && id >= m.pre.chunks[c + 1].wg_base) ++c;
  const ChunkDesc& ch = m.pre.chunks[c];
  const int local = id - ch.wg_base;
  PrefillArgs pa{};
  pa.out = ch.out;
  pa.q = ch.q;
  pa.k = m.pre.k;
  pa.v = m.pre.v;
  pa.table = ch.table;
  pa.ctx_start = ch.ctx_start;
  pa.C = ch.C;
  pa.Hq = m.pre.Hq;
  pa.Hkv = m.pre.Hkv;
  pa.num_blocks = m.pre.num_blocks;
  pa.scale_log2 = m.pre.scale_log2;
  prefill_valu_part<DT_OUT, D>(pa, local % m.pre.Hq, local / m.pre.Hq);
}

// Chunks of the fp32 launch: Hq * C workgroups each, one after another from wg on.
inline int pack_valu_chunks(const char* fn, ChunkSet& cs, int64_t& wg, void* pre_out, const void* pre_query,
                            const int32_t* pre_block_tables, int32_t pre_max_blocks, const int32_t* host_ctx_starts,
                            const int32_t* host_chunk_lens, int32_t num_chunks, int32_t head_dim) {
  const int64_t row_bytes = static_cast<int64_t>(cs.Hq) * head_dim * 4;
  int64_t row0 = 0;
  int n = 0;
  for (int i = 0; i < num_chunks; ++i) {
    const int32_t start = host_ctx_starts[i], C = host_chunk_lens[i];
    if (start < 0 || C < 0) return fail(PKV_EINVAL, "%s: chunk %d has a negative start or length", fn, i);
    if (static_cast<int64_t>(start) + C > static_cast<int64_t>(pre_max_blocks) * kBlock)
      return fail(PKV_EINVAL, "%s: chunk %d extends past pre_max_blocks * block_size", fn, i);
    if (C > 0) {
      ChunkDesc& d = cs.chunks[n++];
      d.out = static_cast<uint8_t*>(pre_out) + row0 * row_bytes;
      d.q = static_cast<const uint8_t*>(pre_query) + row0 * row_bytes;
      d.table = pre_block_tables + static_cast<int64_t>(i) * pre_max_blocks;
      d.ctx_start = start;
      d.C = C;
      d.row_tiles = 0;
      d.wg_base = static_cast<int32_t>(std::min<int64_t>(wg, INT32_MAX));
      wg += static_cast<int64_t>(cs.Hq) * C;
    }
    row0 += C;
  }
  cs.n_chunks = n;
  if (wg > INT32_MAX / 64) return fail(PKV_EINVAL, "%s: too much work for one launch", fn);
  return PKV_OK;
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int paged_attention_mixed(void* dec_out, const void* dec_query, const int32_t* dec_block_tables,
                                     const int32_t* dec_context_lens, int32_t B_dec, int32_t dec_max_blocks,
                                     int32_t dec_max_context_len, const int32_t* host_dec_context_lens,
                                     int32_t dec_partition_size, int32_t dec_group_size, void* workspace,
                                     size_t workspace_bytes, void* pre_out, const void* pre_query,
                                     const int32_t* pre_block_tables, int32_t pre_max_blocks,
                                     const int32_t* host_ctx_starts, const int32_t* host_chunk_lens,
                                     int32_t num_chunks, int32_t out_dtype, const void* k_cache, const void* v_cache,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                     int32_t num_blocks, float scale, int32_t dtype, pkv_stream_t stream) {
  const char* fn = "paged_attention_mixed";
  if (dtype != PKV_BF16 && dtype != PKV_F16 && dtype != PKV_F32)
    return fail(PKV_EUNSUPPORTED, "%s: dtype %d (bf16, fp16 or fp32)", fn, dtype);
  if (out_dtype != PKV_F32 && out_dtype != dtype)
    return fail(PKV_EINVAL, "%s: out_dtype must be PKV_F32 or the input dtype", fn);
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
  if (dtype == PKV_F32 && dec_group_size != 1)
    return fail(PKV_EUNSUPPORTED, "%s: fp32 caches take dec_group_size 1", fn);
  if (dec_group_size != 1 && dec_group_size != mixed_group_size(G))
    return fail(PKV_EUNSUPPORTED, "%s: dec_group_size %d (1, or %d for %d query heads per KV head)", fn,
                dec_group_size, mixed_group_size(G), G);
  if (!k_cache || !v_cache) return fail(PKV_EINVAL, "%s: NULL cache", fn);
  if (num_chunks > 0 && (!pre_out || !pre_query || !pre_block_tables || !host_ctx_starts || !host_chunk_lens))
    return fail(PKV_EINVAL, "%s: NULL prefill pointer", fn);
  // The decode part: paged_attention_decode's argument rules (partition size, workspace, sizes).
  const bool has_dec = B_dec > 0 && dec_max_context_len > 0;
  if (B_dec > 0) {
    const int st = validate(fn, dec_out, out_dtype, dec_query, k_cache, v_cache, dec_block_tables, dec_context_lens,
                            B_dec, num_q_heads, num_kv_heads, head_dim, block_size, dec_max_blocks, num_blocks,
                            dec_max_context_len, dec_partition_size, workspace, workspace_bytes, dtype);
    if (st != PKV_OK) return st;
  }
  if ((reinterpret_cast<uintptr_t>(pre_query) | reinterpret_cast<uintptr_t>(k_cache) |
       reinterpret_cast<uintptr_t>(v_cache)) % 16 != 0)
    return fail(PKV_EINVAL, "%s: queries and caches must be 16-byte aligned", fn);
  MixedArgs m{};
  m.pre.k = k_cache;
  m.pre.v = v_cache;
  m.pre.Hq = num_q_heads;
  m.pre.Hkv = num_kv_heads;
  m.pre.num_blocks = num_blocks;
  m.pre.scale_log2 = scale * kLog2e;
  const Plan pl = make_plan(has_dec ? B_dec : 1, num_q_heads, head_dim, has_dec ? dec_max_context_len : 1,
                            dec_partition_size);
  const int nwd = decode_waves(dec_partition_size, pl);
  m.B_dec = has_dec ? B_dec : 0;
  DecodeArgs& a = m.dec;
  a.out = dec_out;
  a.q = dec_query;
  a.k = k_cache;
  a.v = v_cache;
  a.tables = dec_block_tables;
  a.lens = dec_context_lens;
  a.part_ml = pl.need_bytes ? static_cast<float*>(workspace) : nullptr;
  a.part_o = pl.need_bytes ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + pl.ml_bytes) : nullptr;
  a.Hq = num_q_heads;
  a.Hkv = num_kv_heads;
  a.max_blocks = dec_max_blocks;
  a.num_blocks = num_blocks;
  a.max_parts = pl.max_parts;
  a.part_size = pl.part_size;
  a.scale_log2 = scale * kLog2e;
  if (has_dec && dec_group_size == 1) set_work_order(a, host_dec_context_lens, B_dec, dec_max_context_len, pl);
  if (dtype == PKV_F32) {
    MixedValuArgs mv{};
    mv.dec = a;
    mv.pre = m.pre;
    mv.B_dec = has_dec ? B_dec : 1;
    int64_t wv = has_dec ? static_cast<int64_t>(num_q_heads) * B_dec * pl.max_parts : 0;
    if (wv > INT32_MAX / 64) return fail(PKV_EINVAL, "%s: too much decode work for one launch", fn);
    mv.n_dec_wg = static_cast<int32_t>(wv);
    const int vst = pack_valu_chunks(fn, mv.pre, wv, pre_out, pre_query, pre_block_tables, pre_max_blocks,
                                     host_ctx_starts, host_chunk_lens, num_chunks, head_dim);
    if (vst != PKV_OK) return vst;
    if (wv == 0) return PKV_OK;
    hipStream_t s = as_stream(stream);
    if (head_dim == 64)
      hipLaunchKernelGGL((mixed_valu_kernel<PKV_F32, 64>), dim3(static_cast<uint32_t>(wv)), dim3(64), 0, s, mv);
    else
      hipLaunchKernelGGL((mixed_valu_kernel<PKV_F32, 128>), dim3(static_cast<uint32_t>(wv)), dim3(64), 0, s, mv);
    const int st = check_launch(fn);
    if (st != PKV_OK || !has_dec || pl.max_parts <= 1) return st;
    return paged_attention_decode_reduce(dec_out, out_dtype, dec_context_lens, B_dec, num_q_heads, head_dim,
                                         dec_max_context_len, dec_partition_size, workspace, workspace_bytes, stream);
  }
  m.dec_rows = has_dec ? (dec_group_size == 1 ? B_dec : (B_dec + dec_group_size - 1) / dec_group_size) : 1;
  int64_t wg = has_dec ? (static_cast<int64_t>(num_kv_heads) * m.dec_rows * pl.max_parts + 7) / 8 * 8 : 0;
  m.n_dec_wg = static_cast<int32_t>(wg);
  // prefill chunks, rows packed one after another in pre_query / pre_out
  const int pst = pack_chunks(fn, m.pre, wg, pre_out, pre_query, pre_block_tables, pre_max_blocks, host_ctx_starts,
                              host_chunk_lens, num_chunks, head_dim, elem_size(dtype), elem_size(out_dtype));
  if (pst != PKV_OK) return pst;
  if (wg == 0) return PKV_OK;
  hipStream_t s = as_stream(stream);
  const bool f32out = out_dtype == PKV_F32;
  const int grid = static_cast<int>(wg);
  if (dtype == PKV_BF16) {
    if (f32out)
      launch_d<PKV_BF16, PKV_F32>(m, head_dim, dec_group_size, nwd, grid, s);
    else
      launch_d<PKV_BF16, PKV_BF16>(m, head_dim, dec_group_size, nwd, grid, s);
  } else {
    if (f32out)
      launch_d<PKV_F16, PKV_F32>(m, head_dim, dec_group_size, nwd, grid, s);
    else
      launch_d<PKV_F16, PKV_F16>(m, head_dim, dec_group_size, nwd, grid, s);
  }
  const int st = check_launch(fn);
  if (st != PKV_OK || !has_dec || pl.max_parts <= 1) return st;
  return paged_attention_decode_reduce(dec_out, out_dtype, dec_context_lens, B_dec, num_q_heads, head_dim,
                                       dec_max_context_len, dec_partition_size, workspace, workspace_bytes, stream);
}
