// Device-side check of the inputs the host cannot see without a synchronisation.
//
// The attention and append kernels read block tables, context lengths and slots from device
// memory and treat values outside their contract safely (lengths and block ids are clamped, bad
// slots skipped): a bad value gives a wrong number, never an out-of-bounds access.  This entry
// point reports such values instead of silently absorbing them.  It counts them into a
// caller-owned device array on the caller's stream, without synchronising, and it reads only
// inside the arrays it is given, so no input can make it fault.
//
// The contract it checks: [Serving] "Production Serving: Continuous Batching and PagedAttention",
// Step 4 (a sequence's pages are listed in order; token pos lives in page pos // page_size at
// offset pos % page_size of the one tensor indexed by physical page id) and Step 6 (attention
// runs over the stored tokens only).
#include <climits>

#include "device.h"

namespace pkv {
namespace {

// counts: [0] sequences with a length outside [1, max_context_len] or past its table row,
//         [1] block-table entries among those a sequence's length covers that are outside [0, num_blocks),
//         [2] the smallest sequence index with either fault (INT_MAX when none),
//         [3] slot_mapping entries that are neither -1 nor a slot of the pool.
__global__ void __launch_bounds__(64) reset_counts_kernel(int32_t* counts) {
  if (threadIdx.x < 4) counts[threadIdx.x] = threadIdx.x == 2 ? INT_MAX : 0;
}

// One workgroup per sequence; its threads walk the table entries the length covers.
__global__ void __launch_bounds__(256) check_tables_kernel(const int32_t* __restrict__ tables,
                                                           const int32_t* __restrict__ lens, int32_t max_blocks,
                                                           int32_t max_ctx, int32_t num_blocks, int32_t bs,
                                                           int32_t* counts) {
  __shared__ int32_t s_bad;
  const int b = blockIdx.x;
  const int32_t L = lens[b];
  const bool len_ok = L >= 1 && L <= max_ctx && static_cast<int64_t>(L) <= static_cast<int64_t>(max_blocks) * bs;
  // The entries the kernels would read for this length, after their own clamp to the row.
  const int64_t covered = L > 0 ? (static_cast<int64_t>(L) + bs - 1) / bs : 0;
  const int nb = static_cast<int>(covered < max_blocks ? covered : max_blocks);
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  int bad = 0;
  const int32_t* row = tables + static_cast<int64_t>(b) * max_blocks;
  for (int j = threadIdx.x; j < nb; j += blockDim.x) {
    const int32_t id = row[j];
    bad += (id < 0 || id >= num_blocks) ? 1 : 0;
  }
  if (bad) atomicAdd(&s_bad, bad);
  __syncthreads();
  if (threadIdx.x == 0) {
    if (!len_ok) atomicAdd(&counts[0], 1);
    if (s_bad) atomicAdd(&counts[1], s_bad);
    if (!len_ok || s_bad) atomicMin(&counts[2], b);
  }
}

__global__ void __launch_bounds__(256) check_slots_kernel(const int32_t* __restrict__ slots, int32_t T,
                                                          int64_t pool_slots, int32_t* counts) {
  __shared__ int32_t s_bad;
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
  const int64_t t = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t < T) {
    const int32_t s = slots[t];
    if (s != -1 && (s < 0 || s >= pool_slots)) atomicAdd(&s_bad, 1);
  }
  __syncthreads();
  if (threadIdx.x == 0 && s_bad) atomicAdd(&counts[3], s_bad);
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int paged_check_inputs(const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                                  int32_t max_blocks_per_seq, int32_t max_context_len, const int32_t* slot_mapping,
                                  int32_t T, int32_t num_blocks, int32_t block_size, int32_t* counts,
                                  pkv_stream_t stream) {
  const char* fn = "paged_check_inputs";
  if (B < 0 || T < 0 || max_blocks_per_seq < 0 || num_blocks <= 0 || block_size <= 0)
    return fail(PKV_EINVAL, "%s: bad sizes", fn);
  if (!counts) return fail(PKV_EINVAL, "%s: NULL counts", fn);
  if (B > 0 && (!block_tables || !context_lens)) return fail(PKV_EINVAL, "%s: NULL tables or lengths", fn);
  if (T > 0 && !slot_mapping) return fail(PKV_EINVAL, "%s: NULL slot_mapping", fn);
  hipStream_t s = as_stream(stream);
  hipLaunchKernelGGL(reset_counts_kernel, dim3(1), dim3(64), 0, s, counts);
  if (B > 0)
    hipLaunchKernelGGL(check_tables_kernel, dim3(B), dim3(256), 0, s, block_tables, context_lens, max_blocks_per_seq,
                       max_context_len, num_blocks, block_size, counts);
  if (T > 0)
    hipLaunchKernelGGL(check_slots_kernel, dim3((T + 255) / 256), dim3(256), 0, s, slot_mapping, T,
                       static_cast<int64_t>(num_blocks) * block_size, counts);
  return check_launch(fn);
}
