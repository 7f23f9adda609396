// One launch for a whole continuous-batching step's attention: the decode rows of a batch and the
// rows of any number of prefill chunks.
//
// [Chapter] "Continuous batching and PagedAttention", "How the scheduler works", and [Notes]
// "Continuous batching and PagedAttention: serving many users from one GPU", "Prefill gets in the
// way": a step carries the running sequences' decode tokens and, within the token budget, a chunk
// of a new prompt; production servers put both into the same batch.  Here they go into the same
// kernel launch: workgroups [0, n_dec) each run one (KV head, sequence) of the single-pass decode
// (the body of the decode kernel, 8 waves), the rest each run one (16-row tile, KV head) of a
// prefill chunk (the body of the prefill kernel, 8 waves).  Decode work is dispatched first: its
// workgroups stream the cache from HBM while the prefill workgroups, which are bound by the matrix
// and vector units, fill the other compute units; the step needs one attention launch instead of
// two.  Every output is bit for bit the one the separate launches produce (same bodies, same order
// of arithmetic).  LDS is one buffer, used by whichever body the workgroup runs.
#include <algorithm>

#include "decode_part.h"
#include "prefill_tile.h"

namespace pkv {
namespace {

constexpr int kMaxChunks = 16;

struct ChunkDesc {
  void* out;
  const void* q;
  const int32_t* table;
  int32_t ctx_start;
  int32_t C;
  int32_t row_tiles;
  int32_t wg_base;  // first workgroup of this chunk (a multiple of 8)
};

struct MixedArgs {
  DecodeArgs dec;  // the decode batch: single pass (max_parts 1)
  int32_t B_dec;
  int32_t n_dec_wg;  // Hkv * B_dec rounded up to a multiple of 8
  int32_t n_chunks;
  ChunkDesc chunks[kMaxChunks];
  const void* k;
  const void* v;
  int32_t Hq;
  int32_t Hkv;
  int32_t num_blocks;
  float scale_log2;
};

template <int DT, int DT_OUT, int D, int G>
__global__ void __launch_bounds__(512) mixed_kernel(MixedArgs m) {
  static_assert(PrefillShape<G>::NWAVES == 8, "the mixed launch runs 8-wave prefill tiles (group 4 or 8)");
  constexpr int kDec = decode_smem_floats<D, G, 8>();
  constexpr int kPre = prefill_smem_floats<D, G>();
  __shared__ float smem[kDec > kPre ? kDec : kPre];
  const int id = blockIdx.x;
  if (id < m.n_dec_wg) {
    const int g = id % m.Hkv;
    const int y = id / m.Hkv;
    if (y >= m.B_dec) return;  // padding up to a multiple of 8
    decode_mfma_part<DT, DT_OUT, D, G, 8, false>(m.dec, g, y, 0, smem);
    return;
  }
  int c = 0;
  while (c + 1 < m.n_chunks && id >= m.chunks[c + 1].wg_base) ++c;
  const ChunkDesc& ch = m.chunks[c];
  const int local = id - ch.wg_base;
  if (local >= ch.row_tiles * m.Hkv) return;  // padding up to a multiple of 8
  PrefillArgs pa;
  pa.out = ch.out;
  pa.q = ch.q;
  pa.k = m.k;
  pa.v = m.v;
  pa.table = ch.table;
  pa.ctx_start = ch.ctx_start;
  pa.C = ch.C;
  pa.Hq = m.Hq;
  pa.Hkv = m.Hkv;
  pa.num_blocks = m.num_blocks;
  pa.row_tiles = ch.row_tiles;
  pa.scale_log2 = m.scale_log2;
  prefill_tile<DT, DT_OUT, D, G>(pa, local, smem);
}

template <int DT, int DT_OUT, int D>
void launch_mixed(const MixedArgs& m, int grid, hipStream_t s) {
  if (m.Hq / m.Hkv == 4)
    hipLaunchKernelGGL((mixed_kernel<DT, DT_OUT, D, 4>), dim3(grid), dim3(512), 0, s, m);
  else
    hipLaunchKernelGGL((mixed_kernel<DT, DT_OUT, D, 8>), dim3(grid), dim3(512), 0, s, m);
}

template <int DT, int DT_OUT>
void launch_mixed_d(const MixedArgs& m, int D, int grid, hipStream_t s) {
  if (D == 64)
    launch_mixed<DT, DT_OUT, 64>(m, grid, s);
  else
    launch_mixed<DT, DT_OUT, 128>(m, grid, s);
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int paged_attention_mixed(void* dec_out, const void* dec_query, const int32_t* dec_block_tables,
                                     const int32_t* dec_context_lens, int32_t B_dec, int32_t dec_max_blocks,
                                     int32_t dec_max_context_len, const int32_t* host_dec_context_lens,
                                     void* pre_out, const void* pre_query, const int32_t* pre_block_tables,
                                     int32_t pre_max_blocks, const int32_t* host_ctx_starts,
                                     const int32_t* host_chunk_lens, int32_t num_chunks, int32_t out_dtype,
                                     const void* k_cache, const void* v_cache, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                     float scale, int32_t dtype, pkv_stream_t stream) {
  const char* fn = "paged_attention_mixed";
  if (dtype != PKV_BF16 && dtype != PKV_F16) return fail(PKV_EUNSUPPORTED, "%s: dtype %d (bf16 or fp16)", fn, dtype);
  if (out_dtype != PKV_F32 && out_dtype != dtype)
    return fail(PKV_EINVAL, "%s: out_dtype must be PKV_F32 or the input dtype", fn);
  if (B_dec < 0 || num_chunks < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 || block_size <= 0 ||
      dec_max_blocks < 0 || pre_max_blocks < 0 || dec_max_context_len < 0)
    return fail(PKV_EINVAL, "%s: bad sizes", fn);
  if (num_q_heads % num_kv_heads != 0) return fail(PKV_EINVAL, "%s: num_q_heads not a multiple of num_kv_heads", fn);
  const int G = num_q_heads / num_kv_heads;
  if (G != 4 && G != 8) return fail(PKV_EUNSUPPORTED, "%s: group size %d (the mixed launch takes 4 or 8)", fn, G);
  if (block_size != kBlock) return fail(PKV_EUNSUPPORTED, "%s: block_size %d (kernels implement 16)", fn, block_size);
  if (head_dim != 64 && head_dim != 128) return fail(PKV_EUNSUPPORTED, "%s: head_dim %d", fn, head_dim);
  if (num_chunks > kMaxChunks) return fail(PKV_EUNSUPPORTED, "%s: more than %d prefill chunks", fn, kMaxChunks);
  if (B_dec > kMaxOrder) return fail(PKV_EUNSUPPORTED, "%s: more than %d decode sequences", fn, kMaxOrder);
  if (static_cast<int64_t>(dec_max_context_len) > static_cast<int64_t>(dec_max_blocks) * kBlock)
    return fail(PKV_EINVAL, "%s: dec_max_context_len exceeds dec_max_blocks * block_size", fn);
  if (!k_cache || !v_cache) return fail(PKV_EINVAL, "%s: NULL cache", fn);
  if (B_dec > 0 && (!dec_out || !dec_query || !dec_block_tables || !dec_context_lens))
    return fail(PKV_EINVAL, "%s: NULL decode pointer", fn);
  if (num_chunks > 0 && (!pre_out || !pre_query || !pre_block_tables || !host_ctx_starts || !host_chunk_lens))
    return fail(PKV_EINVAL, "%s: NULL prefill pointer", fn);
  if ((reinterpret_cast<uintptr_t>(dec_query) | reinterpret_cast<uintptr_t>(pre_query) |
       reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(v_cache)) % 16 != 0)
    return fail(PKV_EINVAL, "%s: queries and caches must be 16-byte aligned", fn);
  MixedArgs m{};
  m.k = k_cache;
  m.v = v_cache;
  m.Hq = num_q_heads;
  m.Hkv = num_kv_heads;
  m.num_blocks = num_blocks;
  m.scale_log2 = scale * kLog2e;
  // decode part: the single pass of paged_attention_decode (partition = the longest context)
  const bool has_dec = B_dec > 0 && dec_max_context_len > 0;
  m.B_dec = has_dec ? B_dec : 0;
  DecodeArgs& a = m.dec;
  a.out = dec_out;
  a.q = dec_query;
  a.k = k_cache;
  a.v = v_cache;
  a.tables = dec_block_tables;
  a.lens = dec_context_lens;
  a.Hq = num_q_heads;
  a.Hkv = num_kv_heads;
  a.max_blocks = dec_max_blocks;
  a.num_blocks = num_blocks;
  a.max_parts = 1;
  a.part_size = std::max(kBlock, ((dec_max_context_len + kBlock - 1) / kBlock) * kBlock);
  a.scale_log2 = scale * kLog2e;
  if (has_dec && host_dec_context_lens != nullptr) {
    for (int i = 0; i < B_dec; ++i) a.order[i] = i;
    std::stable_sort(a.order, a.order + B_dec,
                     [&](uint32_t x, uint32_t y) { return host_dec_context_lens[x] > host_dec_context_lens[y]; });
    a.num_order = B_dec;
  }
  int64_t wg = has_dec ? (static_cast<int64_t>(num_kv_heads) * B_dec + 7) / 8 * 8 : 0;
  m.n_dec_wg = static_cast<int32_t>(wg);
  // prefill chunks, rows packed one after another in pre_query / pre_out
  const int64_t row_elems = static_cast<int64_t>(num_q_heads) * head_dim;
  const int es = elem_size(dtype);
  const int oes = elem_size(out_dtype);
  int64_t row0 = 0;
  int n = 0;
  for (int i = 0; i < num_chunks; ++i) {
    const int32_t cs = host_ctx_starts[i], C = host_chunk_lens[i];
    if (cs < 0 || C < 0) return fail(PKV_EINVAL, "%s: chunk %d has a negative start or length", fn, i);
    if (static_cast<int64_t>(cs) + C > static_cast<int64_t>(pre_max_blocks) * kBlock)
      return fail(PKV_EINVAL, "%s: chunk %d extends past pre_max_blocks * block_size", fn, i);
    if (C > 0) {
      ChunkDesc& d = m.chunks[n++];
      d.out = static_cast<uint8_t*>(pre_out) + row0 * row_elems * oes;
      d.q = static_cast<const uint8_t*>(pre_query) + row0 * row_elems * es;
      d.table = pre_block_tables + static_cast<int64_t>(i) * pre_max_blocks;
      d.ctx_start = cs;
      d.C = C;
      d.row_tiles = (C + 15) / 16;
      d.wg_base = static_cast<int32_t>(wg);
      wg += (static_cast<int64_t>(d.row_tiles) * num_kv_heads + 7) / 8 * 8;
    }
    row0 += C;
  }
  m.n_chunks = n;
  if (wg > INT32_MAX) return fail(PKV_EINVAL, "%s: too much work for one launch", fn);
  if (wg == 0) return PKV_OK;
  hipStream_t s = as_stream(stream);
  const bool f32out = out_dtype == PKV_F32;
  if (dtype == PKV_BF16) {
    if (f32out)
      launch_mixed_d<PKV_BF16, PKV_F32>(m, head_dim, static_cast<int>(wg), s);
    else
      launch_mixed_d<PKV_BF16, PKV_BF16>(m, head_dim, static_cast<int>(wg), s);
  } else {
    if (f32out)
      launch_mixed_d<PKV_F16, PKV_F32>(m, head_dim, static_cast<int>(wg), s);
    else
      launch_mixed_d<PKV_F16, PKV_F16>(m, head_dim, static_cast<int>(wg), s);
  }
  return check_launch(fn);
}
