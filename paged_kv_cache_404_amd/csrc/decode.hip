// Paged decode attention: block-table gather, scaled Q.K, online softmax, P.V, GQA groups, and a
// split-K partition + log-sum-exp reduce for long contexts.
//
// What is computed ([Serving] "Production Serving: Continuous Batching and PagedAttention", The
// Build, Step 6): for each sequence b and query head h, every cached token t < L_b is scored
// s_t = scale * <q_{b,h}, K_{g,t}> against KV head g = h / (Hq / Hkv); the scores are
// softmaxed and the output is sum_t w_t V_{g,t}.  Tokens are found through the block table;
// the unused tail of the last block is skipped, never multiplied by zero (stale slots may hold
// NaN).
//
// Split-K: the context is cut into fixed partitions of `part_size` tokens (boundaries depend on
// the position only).  Each partition keeps the usual online-softmax state (reference maximum m,
// sum l, unnormalised output o); partitions of one (sequence, head) are merged exactly:
// M = max_p m_p, out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p.
//
// MI355X mapping (bf16 / fp16): one wavefront handles 32 tokens (two 16-token blocks) of one KV
// head per step.  The GQA group's query rows share every K/V tile load.  Both products run on the
// matrix cores with v_mfma_f32_16x16x32_{bf16,f16}:
//   S^T[token][head] = K[token][:] . Q[head][:]      (A = K rows, B = Q^T, heads padded to 16)
//   O[row][d]       += P[row][token] . V[token][d]    (A = P rows, B = V^T tile)
// The V tile of a (block, head) is stored [token half][D][8 tokens], so that eight consecutive
// tokens of one dimension are one 16-byte load, which is what the P.V operand wants, and sixteen
// dimensions of one half are 256 contiguous bytes.  The softmax weights are
// fed as two 16-bit rows, hi = round(p) and lo = round(p - hi), in the padding rows of the same
// MFMA, so P.V keeps ~16 mantissa bits at no extra matrix instruction.  Scores use exp2 with
// log2(e) folded into the scale; the running maximum is only raised when a score exceeds it by
// more than 2^8 (lazy rescaling: exact, and p stays <= 256), which makes rescaling rare.
#include <algorithm>
#include <cmath>
#include <mutex>
#include <type_traits>

#include "decode_host.h"
#include "decode_part.h"
#include "decode_valu.h"

namespace pkv {
namespace {

template <int DT, int DT_OUT, int D, int G, int NW, bool NEWTOK>
__global__ void __launch_bounds__(NW * 64) decode_mfma_kernel(DecodeArgs a) {
  __shared__ float smem[decode_smem_floats<D, G, NW>()];
  decode_mfma_part<DT, DT_OUT, D, G, NW, NEWTOK>(a, blockIdx.x, blockIdx.y, blockIdx.z, smem);
}

template <int DT, int DT_OUT, int D>
__global__ void __launch_bounds__(64) decode_valu_kernel(DecodeArgs a) {
  decode_valu_part<DT, DT_OUT, D>(a, blockIdx.x, blockIdx.y, blockIdx.z);
}

// ------------------------------------------------------------------------------------------
// Log-sum-exp merge of partitions.  grid = (Hq, B), D threads (D = 64 or 128, so the partials'
// offsets are constants).  MAXP >= max_parts (up to 64).  The context length comes first: rows
// of single-partition sequences were written by the partition pass and end here, and the others
// read only their own partitions' partials, all at once (one dimension of every partial per
// thread).  The maximum over the partitions and each partition's weight are formed once per
// workgroup; the sums run over the partitions in order, as in the loop form below.
// ------------------------------------------------------------------------------------------
template <int DT_OUT, int MAXP, int D>
__global__ void __launch_bounds__(D) decode_reduce_kernel(void* __restrict__ out, const float* __restrict__ part_ml,
                                                          const float* __restrict__ part_o,
                                                          const int32_t* __restrict__ lens, int32_t Hq,
                                                          int32_t max_parts, int32_t part_size) {
  static_assert(MAXP <= D && MAXP <= 64, "one lane of the first wave per partition for (m, l)");
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int d = threadIdx.x;
  const int L = min(lens[b], max_parts * part_size);
  const int nparts = (L + part_size - 1) / part_size;
  if (nparts <= 1) return;  // uniform over the workgroup
  const int64_t row0 = (static_cast<int64_t>(b) * Hq + h) * max_parts;
  const float* __restrict__ po = part_o + row0 * D;  // this row's partials, partition-major
  // Lane p of the first wave fetches partition p's (m, l); every thread fetches its dimension of
  // every partial (slots past the sequence's own partitions re-read its last one: one load per
  // slot, no branch, no extra line).
  float pm = -INFINITY, pl = 0.f;
  if (d < nparts) {
    pm = part_ml[(row0 + d) * 2];
    pl = part_ml[(row0 + d) * 2 + 1];
  }
  float o[MAXP];
#pragma unroll
  for (int p = 0; p < MAXP; ++p) o[p] = po[min(p, nparts - 1) * D + d];
  // The first wave forms the maximum of the partitions' maxima and each partition's weight
  // exp2(m_p - M) once; every thread then sums over the partitions in order.
  __shared__ float sf[MAXP], sl[MAXP];
  if (d < 64) {
    const bool in = d < MAXP && d < nparts;
    const float M = wave_max(in ? pm : -INFINITY);
    if (d < MAXP) {
      sf[d] = in ? fast_exp2(pm - M) : 0.f;
      sl[d] = in ? pl : 0.f;
    }
  }
  __syncthreads();
  float acc = 0.f, lsum = 0.f;
#pragma unroll
  for (int p = 0; p < MAXP; ++p) {
    if (p < nparts) {
      const float f = sf[p];
      acc += f * o[p];
      lsum += f * sl[p];
    }
  }
  store_from_float<DT_OUT>(out, (static_cast<int64_t>(b) * Hq + h) * D + d, acc / lsum);
}

// Any number of partitions: the same merge, 64 partitions at a time (M first, over all of them;
// then each slice's weights formed once and its partials requested at once, the sums in order).
template <int DT_OUT, int D>
__global__ void __launch_bounds__(D) decode_reduce_loop_kernel(void* __restrict__ out,
                                                               const float* __restrict__ part_ml,
                                                               const float* __restrict__ part_o,
                                                               const int32_t* __restrict__ lens, int32_t Hq,
                                                               int32_t max_parts, int32_t part_size) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int d = threadIdx.x;
  const int L = min(lens[b], max_parts * part_size);
  const int nparts = (L + part_size - 1) / part_size;
  if (nparts <= 1) return;  // uniform over the workgroup
  const int64_t row0 = (static_cast<int64_t>(b) * Hq + h) * max_parts;
  __shared__ float sf[64], sl[64], sM;
  if (d < 64) {
    float x = -INFINITY;
    for (int p = d; p < nparts; p += 64) x = fmaxf(x, part_ml[(row0 + p) * 2]);
    x = wave_max(x);
    if (d == 0) sM = x;
  }
  __syncthreads();
  const float M = sM;
  float acc = 0.f, lsum = 0.f;
  for (int p0 = 0; p0 < nparts; p0 += 64) {
    const int cnt = min(64, nparts - p0);
    const float* __restrict__ po = part_o + (row0 + p0) * D;
    float o[64];
#pragma unroll
    for (int p = 0; p < 64; ++p) o[p] = po[min(p, cnt - 1) * D + d];
    if (d < 64) {
      const bool in = d < cnt;
      sf[d] = in ? fast_exp2(part_ml[(row0 + p0 + d) * 2] - M) : 0.f;
      sl[d] = in ? part_ml[(row0 + p0 + d) * 2 + 1] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 64; ++p) {
      if (p < cnt) {
        const float f = sf[p];
        acc += f * o[p];
        lsum += f * sl[p];
      }
    }
    __syncthreads();  // sf and sl are rewritten by the next slice
  }
  store_from_float<DT_OUT>(out, (static_cast<int64_t>(b) * Hq + h) * D + d, acc / lsum);
}

// ------------------------------------------------------------------------------------------
// Host side
// ------------------------------------------------------------------------------------------
template <int DT, int DT_OUT, int D>
int launch_valu(const DecodeArgs& a, int B, hipStream_t s) {
  hipLaunchKernelGGL((decode_valu_kernel<DT, DT_OUT, D>), dim3(a.Hq, B, a.max_parts), dim3(64), 0, s, a);
  return PKV_OK;
}

// Waves per workgroup: decode_waves (decode_host.h).
template <int DT, int DT_OUT, int D, int G>
int launch_mfma(const DecodeArgs& a, int B, int nw, hipStream_t s) {
  const dim3 grid(a.Hkv, B, a.max_parts);
  const bool fused = a.new_k != nullptr;
  if (nw == 4) {
    if (fused)
      hipLaunchKernelGGL((decode_mfma_kernel<DT, DT_OUT, D, G, 4, true>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((decode_mfma_kernel<DT, DT_OUT, D, G, 4, false>), grid, dim3(256), 0, s, a);
  } else {
    if (fused)
      hipLaunchKernelGGL((decode_mfma_kernel<DT, DT_OUT, D, G, 8, true>), grid, dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL((decode_mfma_kernel<DT, DT_OUT, D, G, 8, false>), grid, dim3(512), 0, s, a);
  }
  return PKV_OK;
}

template <int DT, int DT_OUT, int D>
int dispatch_group(const DecodeArgs& a, int B, int nw, hipStream_t s) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_mfma<DT, DT_OUT, D, 1>(a, B, nw, s);
    case 2: return launch_mfma<DT, DT_OUT, D, 2>(a, B, nw, s);
    case 4: return launch_mfma<DT, DT_OUT, D, 4>(a, B, nw, s);
    default: return launch_mfma<DT, DT_OUT, D, 8>(a, B, nw, s);
  }
}

template <int DT, int DT_OUT>
int dispatch_dim(const DecodeArgs& a, int D, int B, int nw, hipStream_t s) {
  if constexpr (DT == PKV_F32) {
    return D == 64 ? launch_valu<DT, DT_OUT, 64>(a, B, s) : launch_valu<DT, DT_OUT, 128>(a, B, s);
  } else {
    return D == 64 ? dispatch_group<DT, DT_OUT, 64>(a, B, nw, s)
                   : dispatch_group<DT, DT_OUT, 128>(a, B, nw, s);
  }
}

int launch_partitions(const DecodeArgs& a, int32_t dtype, int32_t out_dtype, int D, int B, int nw, hipStream_t s) {
  const bool f32out = out_dtype == PKV_F32;
  switch (dtype) {
    case PKV_BF16:
      return f32out ? dispatch_dim<PKV_BF16, PKV_F32>(a, D, B, nw, s)
                    : dispatch_dim<PKV_BF16, PKV_BF16>(a, D, B, nw, s);
    case PKV_F16:
      return f32out ? dispatch_dim<PKV_F16, PKV_F32>(a, D, B, nw, s)
                    : dispatch_dim<PKV_F16, PKV_F16>(a, D, B, nw, s);
    default:
      return dispatch_dim<PKV_F32, PKV_F32>(a, D, B, nw, s);
  }
}

template <int DT_OUT, int D>
void launch_reduce_d(void* out, const float* ml, const float* po, const int32_t* lens, int B, int Hq, int max_parts,
                     int part_size, hipStream_t s) {
  const dim3 grid(Hq, B), block(D);
  if (max_parts <= 4)
    hipLaunchKernelGGL((decode_reduce_kernel<DT_OUT, 4, D>), grid, block, 0, s, out, ml, po, lens, Hq, max_parts,
                       part_size);
  else if (max_parts <= 8)
    hipLaunchKernelGGL((decode_reduce_kernel<DT_OUT, 8, D>), grid, block, 0, s, out, ml, po, lens, Hq, max_parts,
                       part_size);
  else if (max_parts <= 16)
    hipLaunchKernelGGL((decode_reduce_kernel<DT_OUT, 16, D>), grid, block, 0, s, out, ml, po, lens, Hq, max_parts,
                       part_size);
  else if (max_parts <= 32)
    hipLaunchKernelGGL((decode_reduce_kernel<DT_OUT, 32, D>), grid, block, 0, s, out, ml, po, lens, Hq, max_parts,
                       part_size);
  else
    hipLaunchKernelGGL((decode_reduce_kernel<DT_OUT, 64, D>), grid, block, 0, s, out, ml, po, lens, Hq, max_parts,
                       part_size);
}

template <int DT_OUT>
void launch_reduce_t(void* out, const float* ml, const float* po, const int32_t* lens, int B, int Hq, int D,
                     int max_parts, int part_size, hipStream_t s) {
  const dim3 grid(Hq, B);
  if (max_parts <= 64 && D == 64)
    launch_reduce_d<DT_OUT, 64>(out, ml, po, lens, B, Hq, max_parts, part_size, s);
  else if (max_parts <= 64 && D == 128)
    launch_reduce_d<DT_OUT, 128>(out, ml, po, lens, B, Hq, max_parts, part_size, s);
  else if (D == 64)
    hipLaunchKernelGGL((decode_reduce_loop_kernel<DT_OUT, 64>), grid, dim3(64), 0, s, out, ml, po, lens, Hq,
                       max_parts, part_size);
  else
    hipLaunchKernelGGL((decode_reduce_loop_kernel<DT_OUT, 128>), grid, dim3(128), 0, s, out, ml, po, lens, Hq,
                       max_parts, part_size);
}

int launch_reduce(void* out, int32_t out_dtype, const float* ml, const float* po, const int32_t* lens, int B, int Hq,
                  int D, int max_parts, int part_size, hipStream_t s) {
  switch (out_dtype) {
    case PKV_BF16: launch_reduce_t<PKV_BF16>(out, ml, po, lens, B, Hq, D, max_parts, part_size, s); break;
    case PKV_F16: launch_reduce_t<PKV_F16>(out, ml, po, lens, B, Hq, D, max_parts, part_size, s); break;
    default: launch_reduce_t<PKV_F32>(out, ml, po, lens, B, Hq, D, max_parts, part_size, s); break;
  }
  return PKV_OK;
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" size_t paged_attention_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                                         int32_t max_context_len, int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len <= 0 || partition_size <= 0) return 0;
  return make_plan(num_seqs, num_q_heads, head_dim, max_context_len, partition_size).need_bytes;
}

namespace pkv {
namespace {

// Partition pass shared by the plain and the fused-append entry points (new_k == nullptr: plain).
int partitions_impl(const char* fn, void* out, int32_t out_dtype, const void* query, const void* k_cache,
                    const void* v_cache, const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                    int32_t Hq, int32_t Hkv, int32_t D, int32_t bs, int32_t max_blocks, int32_t num_blocks,
                    int32_t max_ctx, float scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
                    int32_t dtype, const void* new_k, const void* new_v, void* k_out, void* v_out,
                    const int32_t* host_lens, pkv_stream_t stream) {
  int st = validate(fn, out, out_dtype, query, k_cache, v_cache, block_tables, context_lens, B, Hq, Hkv, D, bs,
                    max_blocks, num_blocks, max_ctx, partition_size, workspace, workspace_bytes, dtype);
  if (st != PKV_OK || B == 0 || max_ctx == 0) return st;
  if (new_k != nullptr || new_v != nullptr) {
    if (!new_k || !new_v) return fail(PKV_EINVAL, "%s: NULL new_key or new_value", fn);
    if ((reinterpret_cast<uintptr_t>(new_k) | reinterpret_cast<uintptr_t>(new_v)) % 16 != 0)
      return fail(PKV_EINVAL, "%s: new_key and new_value must be 16-byte aligned", fn);
  }
  const Plan pl = make_plan(B, Hq, D, max_ctx, partition_size);
  DecodeArgs a{};
  a.out = out;
  a.q = query;
  a.k = k_cache;
  a.v = v_cache;
  a.tables = block_tables;
  a.lens = context_lens;
  a.part_ml = pl.need_bytes ? static_cast<float*>(workspace) : nullptr;
  a.part_o = pl.need_bytes ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + pl.ml_bytes) : nullptr;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.max_blocks = max_blocks;
  a.num_blocks = num_blocks;
  a.max_parts = pl.max_parts;
  a.part_size = pl.part_size;
  a.scale_log2 = scale * kLog2e;
  a.new_k = new_k;
  a.new_v = new_v;
  a.k_out = k_out;
  a.v_out = v_out;
  set_work_order(a, host_lens, B, max_ctx, pl);
  launch_partitions(a, dtype, out_dtype, D, B, decode_waves(partition_size, pl), as_stream(stream));
  return check_launch(fn);
}

}  // namespace
}  // namespace pkv

extern "C" int paged_attention_decode_partitions(void* out, int32_t out_dtype, const void* query, const void* k_cache,
                                                 const void* v_cache, const int32_t* block_tables,
                                                 const int32_t* context_lens, int32_t B, int32_t num_q_heads,
                                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                                 int32_t max_blocks_per_seq, int32_t num_blocks,
                                                 int32_t max_context_len, float scale, int32_t partition_size,
                                                 void* workspace, size_t workspace_bytes, int32_t dtype,
                                                 const int32_t* host_context_lens, pkv_stream_t stream) {
  return partitions_impl("paged_attention_decode_partitions", out, out_dtype, query, k_cache, v_cache, block_tables,
                         context_lens, B, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                         num_blocks, max_context_len, scale, partition_size, workspace, workspace_bytes, dtype,
                         nullptr, nullptr, nullptr, nullptr, host_context_lens, stream);
}

extern "C" int paged_attention_decode_append_partitions(
    void* out, int32_t out_dtype, const void* query, const void* new_key, const void* new_value, void* k_cache,
    void* v_cache, const int32_t* block_tables, const int32_t* context_lens, int32_t B, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
    int32_t max_context_len, float scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
    int32_t dtype, const int32_t* host_context_lens, pkv_stream_t stream) {
  return partitions_impl("paged_attention_decode_append_partitions", out, out_dtype, query, k_cache, v_cache,
                         block_tables, context_lens, B, num_q_heads, num_kv_heads, head_dim, block_size,
                         max_blocks_per_seq, num_blocks, max_context_len, scale, partition_size, workspace,
                         workspace_bytes, dtype, new_key, new_value, k_cache, v_cache, host_context_lens, stream);
}

extern "C" int paged_attention_decode_reduce(void* out, int32_t out_dtype, const int32_t* context_lens, int32_t B,
                                             int32_t num_q_heads, int32_t head_dim, int32_t max_context_len,
                                             int32_t partition_size, const void* workspace, size_t workspace_bytes,
                                             pkv_stream_t stream) {
  if (B < 0 || num_q_heads <= 0 || (head_dim != 64 && head_dim != 128) || max_context_len < 0 ||
      partition_size < PKV_SINGLE_PASS_ADAPTIVE)
    return fail(PKV_EINVAL, "paged_attention_decode_reduce: bad sizes");
  if (out_dtype != PKV_F32 && out_dtype != PKV_F16 && out_dtype != PKV_BF16)
    return fail(PKV_EINVAL, "paged_attention_decode_reduce: unknown out_dtype %d", out_dtype);
  if (partition_size > 0 && partition_size % kBlock != 0)
    return fail(PKV_EINVAL, "paged_attention_decode_reduce: partition_size must be a multiple of 16");
  if (B == 0 || max_context_len == 0 || partition_size <= 0) return PKV_OK;
  const Plan pl = make_plan(B, num_q_heads, head_dim, max_context_len, partition_size);
  if (pl.max_parts <= 1) return PKV_OK;
  if (!out || !context_lens || !workspace || workspace_bytes < pl.need_bytes)
    return fail(PKV_EINVAL, "paged_attention_decode_reduce: NULL pointer or workspace too small");
  const float* ml = static_cast<const float*>(workspace);
  const float* po = reinterpret_cast<const float*>(static_cast<const uint8_t*>(workspace) + pl.ml_bytes);
  launch_reduce(out, out_dtype, ml, po, context_lens, B, num_q_heads, head_dim, pl.max_parts, pl.part_size,
                as_stream(stream));
  return check_launch("paged_attention_decode_reduce");
}

extern "C" int paged_attention_decode(void* out, int32_t out_dtype, const void* query, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                                      int32_t B, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                                      int32_t max_context_len, float scale, int32_t partition_size, void* workspace,
                                      size_t workspace_bytes, int32_t dtype, const int32_t* host_context_lens,
                                      pkv_stream_t stream) {
  int st = paged_attention_decode_partitions(out, out_dtype, query, k_cache, v_cache, block_tables, context_lens, B,
                                             num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                                             num_blocks, max_context_len, scale, partition_size, workspace,
                                             workspace_bytes, dtype, host_context_lens, stream);
  if (st != PKV_OK) return st;
  return paged_attention_decode_reduce(out, out_dtype, context_lens, B, num_q_heads, head_dim, max_context_len,
                                       partition_size, workspace, workspace_bytes, stream);
}

extern "C" int paged_attention_decode_append(void* out, int32_t out_dtype, const void* query, const void* new_key,
                                             const void* new_value, void* k_cache, void* v_cache,
                                             const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                             int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                                             int32_t max_context_len, float scale, int32_t partition_size,
                                             void* workspace, size_t workspace_bytes, int32_t dtype,
                                             const int32_t* host_context_lens, pkv_stream_t stream) {
  int st = paged_attention_decode_append_partitions(out, out_dtype, query, new_key, new_value, k_cache, v_cache,
                                                    block_tables, context_lens, B, num_q_heads, num_kv_heads,
                                                    head_dim, block_size, max_blocks_per_seq, num_blocks,
                                                    max_context_len, scale, partition_size, workspace,
                                                    workspace_bytes, dtype, host_context_lens, stream);
  if (st != PKV_OK) return st;
  return paged_attention_decode_reduce(out, out_dtype, context_lens, B, num_q_heads, head_dim, max_context_len,
                                       partition_size, workspace, workspace_bytes, stream);
}

extern "C" int paged_attention_decode_newest_partitions(
    void* out, int32_t out_dtype, const void* query, const void* new_key, const void* new_value, const void* k_cache,
    const void* v_cache, const int32_t* block_tables, const int32_t* context_lens, int32_t B, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
    int32_t max_context_len, float scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
    int32_t dtype, const int32_t* host_context_lens, pkv_stream_t stream) {
  return partitions_impl("paged_attention_decode_newest_partitions", out, out_dtype, query, k_cache, v_cache,
                         block_tables, context_lens, B, num_q_heads, num_kv_heads, head_dim, block_size,
                         max_blocks_per_seq, num_blocks, max_context_len, scale, partition_size, workspace,
                         workspace_bytes, dtype, new_key, new_value, nullptr, nullptr, host_context_lens, stream);
}

extern "C" int paged_attention_decode_newest(void* out, int32_t out_dtype, const void* query, const void* new_key,
                                             const void* new_value, const void* k_cache, const void* v_cache,
                                             const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                             int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                                             int32_t max_context_len, float scale, int32_t partition_size,
                                             void* workspace, size_t workspace_bytes, int32_t dtype,
                                             const int32_t* host_context_lens, pkv_stream_t stream) {
  int st = paged_attention_decode_newest_partitions(out, out_dtype, query, new_key, new_value, k_cache, v_cache,
                                                    block_tables, context_lens, B, num_q_heads, num_kv_heads,
                                                    head_dim, block_size, max_blocks_per_seq, num_blocks,
                                                    max_context_len, scale, partition_size, workspace,
                                                    workspace_bytes, dtype, host_context_lens, stream);
  if (st != PKV_OK) return st;
  return paged_attention_decode_reduce(out, out_dtype, context_lens, B, num_q_heads, head_dim, max_context_len,
                                       partition_size, workspace, workspace_bytes, stream);
}

// ------------------------------------------------------------------------------------------
// paged_attention_decode_noalloc: the split-K workspace comes from a fixed device array of the
// library instead of the caller, for callers that cannot allocate device memory.
// ------------------------------------------------------------------------------------------
namespace pkv {
namespace {

constexpr size_t kScratchBytes = static_cast<size_t>(PKV_NOALLOC_SCRATCH_BYTES);
constexpr int kMaxDevices = 64;

// One copy per GPU, held until the process ends.  In host code the name is only a stand-in for
// the symbol: the device address of each GPU's copy is looked up once (scratch_on_current_device)
// and only that address is handed to kernels.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, looked up on the first call on that
// device (with it current) and kept.
int scratch_on_current_device(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PKV_EHIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(PKV_EUNSUPPORTED, "%s: device %d beyond %d", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(PKV_EHIP, "%s: hipGetSymbolAddress(scratch) on device %d: %s", fn, dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

}  // namespace
}  // namespace pkv

extern "C" int paged_attention_decode_noalloc(void* out, int32_t out_dtype, const void* query, const void* k_cache,
                                              const void* v_cache, const int32_t* block_tables,
                                              const int32_t* context_lens, int32_t B, int32_t num_q_heads,
                                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                              int32_t max_blocks_per_seq, int32_t num_blocks,
                                              int32_t max_context_len, float scale, int32_t partition_size,
                                              int32_t dtype, const int32_t* host_context_lens, pkv_stream_t stream) {
  const char* fn = "paged_attention_decode_noalloc";
  const size_t need = paged_attention_decode_workspace_bytes(B, num_q_heads, head_dim, max_context_len,
                                                             partition_size);
  if (need > kScratchBytes)
    return fail(PKV_EINVAL, "%s: split-K partials need %zu bytes, more than the %zu-byte static scratch", fn, need,
                kScratchBytes);
  // Everything the host can check is checked before the scratch is touched.
  int st = validate(fn, out, out_dtype, query, k_cache, v_cache, block_tables, context_lens, B, num_q_heads,
                    num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, max_context_len,
                    partition_size, nullptr, 0, dtype, /*check_workspace=*/false);
  if (st != PKV_OK || B == 0 || max_context_len == 0) return st;
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_on_current_device(fn, &ws);
    if (st != PKV_OK) return st;
  }
  // The partials need no initial value: every one the reduce reads is written by the partition
  // pass of the same call.
  return paged_attention_decode(out, out_dtype, query, k_cache, v_cache, block_tables, context_lens, B, num_q_heads,
                                num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, max_context_len,
                                scale, partition_size, ws, need ? kScratchBytes : 0, dtype, host_context_lens,
                                stream);
}
