// Prefill chunks of a mixed decode + prefill launch (csrc/mixed.hip over bf16 / fp16 caches,
// csrc/mixed_fp8.hip over the FP8 cache): their descriptors, the prefill role of a workgroup, and
// the host-side packing of the chunks into the grid after the decode workgroups.
#pragma once
#include "prefill_tile.h"
#include "status.h"

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

// What every prefill role shares: the caches (and FP8 scales), head counts and scale.
struct ChunkSet {
  int32_t n_chunks;
  ChunkDesc chunks[kMaxChunks];
  const void* k;
  const void* v;
  const float* ksc;  // FP8 cache only
  const float* vsc;
  int32_t Hq;
  int32_t Hkv;
  int32_t num_blocks;
  float scale_log2;
};

constexpr int smax(int a, int b) { return a > b ? a : b; }

// Workgroup id (at or past the decode workgroups) runs one (16-row tile, KV head) of its chunk.
template <int DT, int DT_OUT, int D, int G, bool FP8>
__device__ __forceinline__ void mixed_prefill_role(const ChunkSet& cs, int id, float* smem) {
  int c = 0;
  while (c + 1 < cs.n_chunks && id >= cs.chunks[c + 1].wg_base) ++c;
  const ChunkDesc& ch = cs.chunks[c];
  const int local = id - ch.wg_base;
  if (local >= ch.row_tiles * cs.Hkv) return;  // padding up to a multiple of 8
  PrefillArgs pa;
  pa.out = ch.out;
  pa.q = ch.q;
  pa.k = cs.k;
  pa.v = cs.v;
  pa.table = ch.table;
  pa.ctx_start = ch.ctx_start;
  pa.C = ch.C;
  pa.Hq = cs.Hq;
  pa.Hkv = cs.Hkv;
  pa.num_blocks = cs.num_blocks;
  pa.row_tiles = ch.row_tiles;
  pa.scale_log2 = cs.scale_log2;
  pa.ksc = cs.ksc;
  pa.vsc = cs.vsc;
  prefill_tile<DT, DT_OUT, D, G, FP8>(pa, local, smem);
}

// Packs the chunks (rows one after another in pre_query / pre_out, elements of q_bytes / o_bytes
// bytes) into cs, each at a multiple of 8 workgroups from wg on; wg ends past the last chunk.
inline int pack_chunks(const char* fn, ChunkSet& cs, int64_t& wg, void* pre_out, const void* pre_query,
                       const int32_t* pre_block_tables, int32_t pre_max_blocks, const int32_t* host_ctx_starts,
                       const int32_t* host_chunk_lens, int32_t num_chunks, int32_t head_dim, int q_bytes,
                       int o_bytes) {
  const int64_t row_elems = static_cast<int64_t>(cs.Hq) * head_dim;
  int64_t row0 = 0;
  int n = 0;
  for (int i = 0; i < num_chunks; ++i) {
    const int32_t start = host_ctx_starts[i], C = host_chunk_lens[i];
    if (start < 0 || C < 0) return fail(PKV_EINVAL, "%s: chunk %d has a negative start or length", fn, i);
    if (static_cast<int64_t>(start) + C > static_cast<int64_t>(pre_max_blocks) * kBlock)
      return fail(PKV_EINVAL, "%s: chunk %d extends past pre_max_blocks * block_size", fn, i);
    if (C > 0) {
      ChunkDesc& d = cs.chunks[n++];
      d.out = static_cast<uint8_t*>(pre_out) + row0 * row_elems * o_bytes;
      d.q = static_cast<const uint8_t*>(pre_query) + row0 * row_elems * q_bytes;
      d.table = pre_block_tables + static_cast<int64_t>(i) * pre_max_blocks;
      d.ctx_start = start;
      d.C = C;
      d.row_tiles = (C + 15) / 16;
      d.wg_base = static_cast<int32_t>(wg);
      wg += (static_cast<int64_t>(d.row_tiles) * cs.Hkv + 7) / 8 * 8;
    }
    row0 += C;
  }
  cs.n_chunks = n;
  if (wg > INT32_MAX) return fail(PKV_EINVAL, "%s: too much work for one launch", fn);
  return PKV_OK;
}

}  // namespace
}  // namespace pkv
