// Host-side planning and argument checks of the decode entry points (csrc/decode.hip,
// csrc/decode_group.hip): split-K workspace layout and the validation every decode call shares.
#pragma once
#include <algorithm>
#include <cstddef>
#include <cstdint>

#include "decode_part.h"
#include "device.h"

namespace pkv {
namespace {

struct Plan {
  int32_t part_size;
  int32_t max_parts;
  size_t ml_bytes;
  size_t need_bytes;
};

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

Plan make_plan(int32_t B, int32_t Hq, int32_t D, int32_t max_ctx, int32_t partition_size) {
  Plan pl{};
  if (partition_size <= 0) {
    pl.part_size = static_cast<int32_t>(((static_cast<int64_t>(max_ctx) + kBlock - 1) / kBlock) * kBlock);
    if (pl.part_size < kBlock) pl.part_size = kBlock;
    pl.max_parts = 1;
    pl.ml_bytes = 0;
    pl.need_bytes = 0;
  } else {
    pl.part_size = partition_size;
    pl.max_parts = static_cast<int32_t>((static_cast<int64_t>(max_ctx) + partition_size - 1) / partition_size);
    pl.ml_bytes = align256(static_cast<size_t>(B) * Hq * pl.max_parts * 2 * sizeof(float));
    pl.need_bytes = pl.ml_bytes + static_cast<size_t>(B) * Hq * pl.max_parts * D * sizeof(float);
  }
  return pl;
}

int validate(const char* fn, void* out, int32_t out_dtype, const void* query, const void* k_cache,
             const void* v_cache, const int32_t* block_tables, const int32_t* context_lens, int32_t B, int32_t Hq,
             int32_t Hkv, int32_t D, int32_t bs, int32_t max_blocks, int32_t num_blocks, int32_t max_ctx,
             int32_t partition_size, const void* workspace, size_t workspace_bytes, int32_t dtype,
             bool check_workspace = true) {
  if (!valid_dtype(dtype)) return fail(PKV_EINVAL, "%s: unknown dtype %d", fn, dtype);
  if (out_dtype != PKV_F32 && out_dtype != dtype)
    return fail(PKV_EINVAL, "%s: out_dtype must be PKV_F32 or the input dtype", fn);
  if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || bs <= 0 || max_blocks < 0 || num_blocks <= 0 || max_ctx < 0)
    return fail(PKV_EINVAL, "%s: bad sizes", fn);
  if (Hq % Hkv != 0) return fail(PKV_EINVAL, "%s: num_q_heads %d not a multiple of num_kv_heads %d", fn, Hq, Hkv);
  if (bs != kBlock) return fail(PKV_EUNSUPPORTED, "%s: block_size %d (kernels implement 16)", fn, bs);
  if (D != 64 && D != 128) return fail(PKV_EUNSUPPORTED, "%s: head_dim %d (64 or 128)", fn, D);
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(PKV_EUNSUPPORTED, "%s: group size %d", fn, G);
  if (B > 65535 || Hq > 65535) return fail(PKV_EUNSUPPORTED, "%s: batch or head count above 65535", fn);
  if (partition_size != PKV_SINGLE_PASS_ADAPTIVE && (partition_size < 0 || partition_size % bs != 0))
    return fail(PKV_EINVAL, "%s: partition_size %d must be 0, -1 or a multiple of block_size", fn, partition_size);
  if (partition_size > 0 && (max_ctx + static_cast<int64_t>(partition_size) - 1) / partition_size > 65535)
    return fail(PKV_EUNSUPPORTED, "%s: more than 65535 partitions per sequence", fn);
  if (static_cast<int64_t>(max_ctx) > static_cast<int64_t>(max_blocks) * bs)
    return fail(PKV_EINVAL, "%s: max_context_len %d exceeds max_blocks_per_seq * block_size", fn, max_ctx);
  if (B == 0) return PKV_OK;
  if (!out || !query || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PKV_EINVAL, "%s: NULL pointer", fn);
  const Plan pl = make_plan(B, Hq, D, max_ctx, partition_size);
  if (check_workspace && pl.need_bytes > 0 && (!workspace || workspace_bytes < pl.need_bytes))
    return fail(PKV_EINVAL, "%s: workspace of %zu bytes needed, %zu given", fn, pl.need_bytes, workspace_bytes);
  const uintptr_t al = reinterpret_cast<uintptr_t>(query) | reinterpret_cast<uintptr_t>(k_cache) |
                       reinterpret_cast<uintptr_t>(v_cache) | reinterpret_cast<uintptr_t>(workspace);
  if (al % 16 != 0) return fail(PKV_EINVAL, "%s: query, caches and workspace must be 16-byte aligned", fn);
  return PKV_OK;
}

// Waves per workgroup of the matrix-core decode: 4 for partitions of up to 512 tokens (<= 4 steps
// per wave), 8 above and for the single pass.  It depends only on the caller's partition_size,
// never on the batch (a single pass spans the batch's longest context, so its wave count is
// fixed): a sequence's reduction order, and so its output bits, do not depend on the rest of the
// batch.  The batch-adaptive single pass (partition_size -1) applies the 512-token rule to the
// batch's longest context instead.
inline int decode_waves(int32_t partition_size, const Plan& pl) {
  return (partition_size != 0 && pl.part_size <= 512) ? 4 : 8;
}

// Work order (largest work first, smallest last) from a host copy of the lengths (B <=
// kMaxOrder; otherwise rows run in batch order): rows sorted by the size of their sequence's last
// partition (the whole context for a single pass), largest first, ties longest first; and each
// sequence's partitions rotated so that its last one falls in the grid's last slice.  Full
// partitions are then all dispatched before the ragged last ones, which go smallest last.  The
// schedule only: every partition's arithmetic is the same wherever it runs.
inline void set_work_order(DecodeArgs& a, const int32_t* host_lens, int32_t B, int32_t max_ctx, const Plan& pl) {
  if (host_lens == nullptr || B > kMaxOrder) return;
  int32_t nparts[kMaxOrder], last[kMaxOrder], idx[kMaxOrder];
  for (int i = 0; i < B; ++i) {
    const int L = std::max(0, std::min(host_lens[i], max_ctx));
    nparts[i] = (L + pl.part_size - 1) / pl.part_size;
    last[i] = L - std::max(0, nparts[i] - 1) * pl.part_size;
    idx[i] = i;
  }
  std::stable_sort(idx, idx + B, [&](int32_t x, int32_t y) {
    return last[x] != last[y] ? last[x] > last[y] : host_lens[x] > host_lens[y];
  });
  for (int i = 0; i < B; ++i) {
    const uint32_t rot = static_cast<uint32_t>(nparts[idx[i]] % pl.max_parts);
    a.order[i] = static_cast<uint32_t>(idx[i]) | (rot << 16);
  }
  a.num_order = B;
}

}  // namespace
}  // namespace pkv
