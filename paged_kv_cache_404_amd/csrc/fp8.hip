// FP8 K/V cache: append with quantisation, and paged decode attention over the quantised cache.
//
// [Notes] "Continuous batching and PagedAttention: serving many users from one GPU", "Memory, not
// compute, caps the batch": the cache bounds how many sequences run at once and a quantised cache
// multiplies the tokens that fit; on a bandwidth-bound decode it also divides the bytes per step.
// Format: OCP 8-bit floating point E4M3 (bias 7, largest finite 448, subnormals, no infinities),
// which gfx950 converts in hardware (v_cvt_pk_fp8_f32, v_cvt_scalef32_pk_{bf16,f16}_fp8).
//
// Quantisation, per (token, KV head) row x of head_dim values (x widened exactly to fp32):
//   amax = max |x_i|,  s = amax / 448 (stored),  inv = 448 / amax (0 when amax = 0),
//   code_i = E4M3 round-to-nearest-even(x_i * inv),  value_i = code_i * s.
// K and V rows are quantised separately; every (block, head, slot) has its own K and V scale, so an
// append never touches the other tokens of its block.
//
// Layout: K tile of one (block, head) = 16 tokens x D bytes, byte (t, d) at
//   ((d / 64) * 2 + (t / 4) % 2) * 512 + ((t / 8) * 4 + t % 4) * 64 + d % 64,
// so that a matrix-core operand load of one token set and 64 dimensions is one 512-byte run per
// block; V tile = [D][16] bytes (dimension-major); scales fp32 [block][head][slot].
//
// Decode (MI355X): the structure of the bf16 kernel (one wave per 32-token step, GQA heads in the
// MFMA columns, hi/lo weights in the padding rows, lazy rescale, one step of loads in flight).
// Codes are widened exactly to bf16/fp16 in registers for v_mfma_f32_16x16x32; a lane's 16-byte K
// load holds dimensions [64p + 16 q4, +16) of one token, split into k-steps 2p and 2p + 1, and the
// query fragments follow the same dimension order.  Per-token scales enter outside the products:
// each score is multiplied by its key's scale, and each weight by its value's scale before P.V
// (the softmax sum uses the unscaled weight).
#include <algorithm>
#include <cmath>

#include "decode_fp8_group.h"
#include "decode_fp8_part.h"

namespace pkv {
namespace {


__host__ __device__ __forceinline__ int fp8_k_pos(int t, int d) {
  return ((d >> 6) * 2 + ((t >> 2) & 1)) * 512 + ((t >> 3) * 4 + (t & 3)) * 64 + (d & 63);
}

template <int DT>
__device__ __forceinline__ float in_elem(const uint8_t* row, int i) {
  if constexpr (DT == PKV_F32) {
    return reinterpret_cast<const float*>(row)[i];
  } else if constexpr (DT == PKV_BF16) {
    return bf16_bits_to_float(reinterpret_cast<const uint16_t*>(row)[i]);
  } else {
    return f16_bits_to_float(reinterpret_cast<const uint16_t*>(row)[i]);
  }
}


// R = D / 8 lanes per (token, head) row; lane j quantises dimensions [8j, 8j + 8).  A workgroup
// takes one head of a window of 256 / R consecutive input tokens, and consecutive windows of a
// head run on the same XCD (workgroup w runs on XCD w % 8; the logical window index is remapped
// so that each XCD owns a contiguous range): the byte-wide V codes of a prompt's block then reach
// one L2, which merges each line before writing it back.
template <int DT_IN, int D>
__global__ void __launch_bounds__(256) append_fp8_kernel(uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
                                                         float* __restrict__ ksc, float* __restrict__ vsc,
                                                         const uint8_t* __restrict__ key,
                                                         const uint8_t* __restrict__ value, int64_t key_stride_b,
                                                         int64_t value_stride_b, const int32_t* __restrict__ slots,
                                                         int32_t T, int32_t H, int32_t num_blocks, int32_t windows) {
  constexpr int R = D / 8;
  constexpr int TW = 256 / R;  // tokens per window
  constexpr int ES = DT_IN == PKV_F32 ? 4 : 2;
  const int64_t per_xcd = gridDim.x / 8;  // the grid is a multiple of 8
  const int64_t logical = static_cast<int64_t>(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  const int j = static_cast<int>(threadIdx.x % R);
  const int64_t tt = (logical % windows) * TW + threadIdx.x / R;
  // Every lane takes part in the row maximum below, so out-of-range lanes stay (inactive).
  const bool active = logical < static_cast<int64_t>(H) * windows && tt < T;
  const int t = active ? static_cast<int>(tt) : 0;
  const int h = active ? static_cast<int>(logical / windows) : 0;
  const int slot = active ? slots[t] : -1;
  const bool ok = slot >= 0 && slot / kBlock < num_blocks;  // -1 = skip; out-of-pool slots are never written
  float kx[8], vx[8];
  float ka = 0.f, va = 0.f;
  const uint8_t* krow = key + t * key_stride_b + (static_cast<int64_t>(h) * D + 8 * j) * ES;
  const uint8_t* vrow = value + t * value_stride_b + (static_cast<int64_t>(h) * D + 8 * j) * ES;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    kx[i] = ok ? in_elem<DT_IN>(krow, i) : 0.f;
    vx[i] = ok ? in_elem<DT_IN>(vrow, i) : 0.f;
    ka = fmaxf(ka, fabsf(kx[i]));
    va = fmaxf(va, fabsf(vx[i]));
  }
  // Row maximum over the row's R lanes (aligned groups inside the wave; every lane takes part).
#pragma unroll
  for (int o = R / 2; o > 0; o >>= 1) {
    ka = fmaxf(ka, __shfl_xor(ka, o));
    va = fmaxf(va, __shfl_xor(va, o));
  }
  if (!ok) return;
  const float ks = __fdiv_rn(ka, kE4M3Max);
  const float vs = __fdiv_rn(va, kE4M3Max);
  const float kinv = ka > 0.f ? __fdiv_rn(kE4M3Max, ka) : 0.f;
  const float vinv = va > 0.f ? __fdiv_rn(kE4M3Max, va) : 0.f;
  const int64_t blk = slot / kBlock;
  const int off = slot % kBlock;
  const int64_t head = blk * H + h;
  u32x2 kw;
  kw[0] = pack4_fp8(kx[0] * kinv, kx[1] * kinv, kx[2] * kinv, kx[3] * kinv);
  kw[1] = pack4_fp8(kx[4] * kinv, kx[5] * kinv, kx[6] * kinv, kx[7] * kinv);
  *reinterpret_cast<u32x2*>(kc + head * kBlock * D + fp8_k_pos(off, 8 * j)) = kw;
  const uint32_t v0 = pack4_fp8(vx[0] * vinv, vx[1] * vinv, vx[2] * vinv, vx[3] * vinv);
  const uint32_t v1 = pack4_fp8(vx[4] * vinv, vx[5] * vinv, vx[6] * vinv, vx[7] * vinv);
  uint8_t* vcol = vc + (head * D + 8 * j) * kBlock + off;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    vcol[i * kBlock] = static_cast<uint8_t>(v0 >> (8 * i));
    vcol[(i + 4) * kBlock] = static_cast<uint8_t>(v1 >> (8 * i));
  }
  if (j == 0) {
    ksc[head * kBlock + off] = ks;
    vsc[head * kBlock + off] = vs;
  }
}

// grid = (Hkv, B, max_parts): the body of decode_fp8_part.h per workgroup.
template <int DT, int DT_OUT, int D, int G, int NW, bool NEWTOK>
__global__ void __launch_bounds__(NW * 64) decode_fp8_kernel(Fp8Args a) {
  __shared__ float smem[fp8_decode_smem_floats<D, G, NW>()];
  decode_fp8_part<DT, DT_OUT, D, G, NW, NEWTOK>(a, blockIdx.x, blockIdx.y, blockIdx.z, smem);
}

// Waves per workgroup as in the bf16 kernel: 4 for partitions of up to 512 tokens, 8 above and for
// the single pass (so the output bits never depend on the rest of the batch); the batch-adaptive
// single pass applies the 512-token rule to the batch's longest context.
template <int DT, int DT_OUT, int D, int G>
void launch_fp8(const Fp8Args& a, int B, bool wide, hipStream_t s) {
  const dim3 grid(a.Hkv, B, a.max_parts);
  const bool fused = a.new_k != nullptr;
  if (wide) {
    if (fused)
      hipLaunchKernelGGL((decode_fp8_kernel<DT, DT_OUT, D, G, 8, true>), grid, dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL((decode_fp8_kernel<DT, DT_OUT, D, G, 8, false>), grid, dim3(512), 0, s, a);
  } else {
    if (fused)
      hipLaunchKernelGGL((decode_fp8_kernel<DT, DT_OUT, D, G, 4, true>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((decode_fp8_kernel<DT, DT_OUT, D, G, 4, false>), grid, dim3(256), 0, s, a);
  }
}

template <int DT, int DT_OUT, int D>
void dispatch_fp8_group(const Fp8Args& a, int B, bool wide, hipStream_t s) {
  switch (a.Hq / a.Hkv) {
    case 1: launch_fp8<DT, DT_OUT, D, 1>(a, B, wide, s); break;
    case 2: launch_fp8<DT, DT_OUT, D, 2>(a, B, wide, s); break;
    case 4: launch_fp8<DT, DT_OUT, D, 4>(a, B, wide, s); break;
    default: launch_fp8<DT, DT_OUT, D, 8>(a, B, wide, s); break;
  }
}

template <int DT, int DT_OUT>
void dispatch_fp8_dim(const Fp8Args& a, int D, int B, bool wide, hipStream_t s) {
  if (D == 64)
    dispatch_fp8_group<DT, DT_OUT, 64>(a, B, wide, s);
  else
    dispatch_fp8_group<DT, DT_OUT, 128>(a, B, wide, s);
}

// Grouped FP8 decode: grid = (Hkv, groups, max_parts); at least two waves per SIMD whatever NW.
template <int DT, int DT_OUT, int D, int G, int NS, int NW>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
decode_fp8_group_kernel(Fp8Args a, int32_t B) {
  __shared__ float smem[fp8_group_smem_floats<D, G, NS, NW>()];
  decode_fp8_group_part<DT, DT_OUT, D, G, NS, NW>(a, B, blockIdx.x, blockIdx.y, blockIdx.z, smem);
}

template <int DT, int DT_OUT, int D, int G, int NS>
void launch_fp8_group_ns(const Fp8Args& a, int B, int ngroups, bool wide, hipStream_t s) {
  const dim3 grid(a.Hkv, ngroups, a.max_parts);
  if (wide)
    hipLaunchKernelGGL((decode_fp8_group_kernel<DT, DT_OUT, D, G, NS, 8>), grid, dim3(512), 0, s, a, B);
  else
    hipLaunchKernelGGL((decode_fp8_group_kernel<DT, DT_OUT, D, G, NS, 4>), grid, dim3(256), 0, s, a, B);
}

// Group sizes whose columns (group_size x query heads per KV head) fill 8 or 16 matrix columns.
template <int DT, int DT_OUT, int D>
bool launch_fp8_group_gs(const Fp8Args& a, int B, int G, int NS, int ngroups, bool wide, hipStream_t s) {
  switch (G * 100 + NS) {
    case 108: launch_fp8_group_ns<DT, DT_OUT, D, 1, 8>(a, B, ngroups, wide, s); return true;
    case 116: launch_fp8_group_ns<DT, DT_OUT, D, 1, 16>(a, B, ngroups, wide, s); return true;
    case 204: launch_fp8_group_ns<DT, DT_OUT, D, 2, 4>(a, B, ngroups, wide, s); return true;
    case 208: launch_fp8_group_ns<DT, DT_OUT, D, 2, 8>(a, B, ngroups, wide, s); return true;
    case 402: launch_fp8_group_ns<DT, DT_OUT, D, 4, 2>(a, B, ngroups, wide, s); return true;
    case 404: launch_fp8_group_ns<DT, DT_OUT, D, 4, 4>(a, B, ngroups, wide, s); return true;
    case 802: launch_fp8_group_ns<DT, DT_OUT, D, 8, 2>(a, B, ngroups, wide, s); return true;
    default: return false;
  }
}

template <int DT, int DT_OUT>
bool launch_fp8_group_dim(const Fp8Args& a, int B, int D, int G, int NS, int ngroups, bool wide, hipStream_t s) {
  return D == 64 ? launch_fp8_group_gs<DT, DT_OUT, 64>(a, B, G, NS, ngroups, wide, s)
                 : launch_fp8_group_gs<DT, DT_OUT, 128>(a, B, G, NS, ngroups, wide, s);
}

int fp8_partitions(const char* fn, void* out, int32_t out_dtype, const void* query, const void* k_cache,
                   const void* v_cache, const void* k_scale, const void* v_scale, const int32_t* block_tables,
                   const int32_t* context_lens, int32_t B, int32_t Hq, int32_t Hkv, int32_t D, int32_t bs,
                   int32_t max_blocks, int32_t num_blocks, int32_t max_ctx, float scale, int32_t partition_size,
                   void* workspace, size_t workspace_bytes, int32_t q_dtype, const int32_t* host_lens,
                   pkv_stream_t stream, const void* new_k = nullptr, const void* new_v = nullptr) {
  Fp8Args a;
  bool wide = false, empty = true;
  const int st = fp8_setup(fn, a, wide, empty, out, out_dtype, query, k_cache, v_cache, k_scale, v_scale,
                           block_tables, context_lens, B, Hq, Hkv, D, bs, max_blocks, num_blocks, max_ctx, scale,
                           partition_size, workspace, workspace_bytes, q_dtype, host_lens, new_k, new_v);
  if (st != PKV_OK || empty) return st;
  hipStream_t s = as_stream(stream);
  const bool f32out = out_dtype == PKV_F32;
  if (q_dtype == PKV_BF16) {
    if (f32out)
      dispatch_fp8_dim<PKV_BF16, PKV_F32>(a, D, B, wide, s);
    else
      dispatch_fp8_dim<PKV_BF16, PKV_BF16>(a, D, B, wide, s);
  } else {
    if (f32out)
      dispatch_fp8_dim<PKV_F16, PKV_F32>(a, D, B, wide, s);
    else
      dispatch_fp8_dim<PKV_F16, PKV_F16>(a, D, B, wide, s);
  }
  return check_launch(fn);
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" int paged_cache_append_fp8(void* k_cache, void* v_cache, void* k_scale, void* v_scale, const void* key,
                                      const void* value, int64_t key_stride, int64_t value_stride,
                                      const int32_t* slot_mapping, int32_t T, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t num_blocks, int32_t in_dtype, pkv_stream_t stream) {
  const char* fn = "paged_cache_append_fp8";
  if (!valid_dtype(in_dtype)) return fail(PKV_EINVAL, "%s: unknown dtype %d", fn, in_dtype);
  if (T < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail(PKV_EINVAL, "%s: bad sizes", fn);
  if (block_size != kBlock) return fail(PKV_EUNSUPPORTED, "%s: block_size %d (16 only)", fn, block_size);
  if (head_dim != 64 && head_dim != 128) return fail(PKV_EUNSUPPORTED, "%s: head_dim %d (64 or 128)", fn, head_dim);
  if (T == 0) return PKV_OK;
  if (!k_cache || !v_cache || !k_scale || !v_scale || !key || !value || !slot_mapping)
    return fail(PKV_EINVAL, "%s: NULL pointer", fn);
  const int es = elem_size(in_dtype);
  const int64_t row = static_cast<int64_t>(num_kv_heads) * head_dim;
  if (key_stride == 0) key_stride = row;
  if (value_stride == 0) value_stride = row;
  if (key_stride < row || value_stride < row) return fail(PKV_EINVAL, "%s: token stride below num_kv_heads*head_dim", fn);
  if ((reinterpret_cast<uintptr_t>(key) | reinterpret_cast<uintptr_t>(value)) % es != 0 ||
      (reinterpret_cast<uintptr_t>(k_cache) | reinterpret_cast<uintptr_t>(k_scale) |
       reinterpret_cast<uintptr_t>(v_scale)) % 8 != 0)
    return fail(PKV_EINVAL, "%s: misaligned pointer", fn);
  const int tw = 256 / (head_dim / 8);  // tokens per workgroup window
  const int64_t windows = (static_cast<int64_t>(T) + tw - 1) / tw;
  const int64_t grid = (static_cast<int64_t>(num_kv_heads) * windows + 7) / 8 * 8;
  if (grid > INT32_MAX || windows > INT32_MAX) return fail(PKV_EINVAL, "%s: too many tokens", fn);
  hipStream_t s = as_stream(stream);
  uint8_t* kc = static_cast<uint8_t*>(k_cache);
  uint8_t* vc = static_cast<uint8_t*>(v_cache);
  float* ks = static_cast<float*>(k_scale);
  float* vs = static_cast<float*>(v_scale);
  const uint8_t* kin = static_cast<const uint8_t*>(key);
  const uint8_t* vin = static_cast<const uint8_t*>(value);
  const dim3 gr(static_cast<uint32_t>(grid)), bl(256);
#define PKV_APPEND_FP8(DT, DD)                                                                                    \
  hipLaunchKernelGGL((append_fp8_kernel<DT, DD>), gr, bl, 0, s, kc, vc, ks, vs, kin, vin, key_stride * es,        \
                     value_stride * es, slot_mapping, T, num_kv_heads, num_blocks, static_cast<int32_t>(windows))
  if (head_dim == 64) {
    if (in_dtype == PKV_BF16)
      PKV_APPEND_FP8(PKV_BF16, 64);
    else if (in_dtype == PKV_F16)
      PKV_APPEND_FP8(PKV_F16, 64);
    else
      PKV_APPEND_FP8(PKV_F32, 64);
  } else {
    if (in_dtype == PKV_BF16)
      PKV_APPEND_FP8(PKV_BF16, 128);
    else if (in_dtype == PKV_F16)
      PKV_APPEND_FP8(PKV_F16, 128);
    else
      PKV_APPEND_FP8(PKV_F32, 128);
  }
#undef PKV_APPEND_FP8
  return check_launch(fn);
}

extern "C" int paged_attention_decode_fp8_partitions(
    void* out, int32_t out_dtype, const void* query, const void* k_cache, const void* v_cache, const void* k_scale,
    const void* v_scale, const int32_t* block_tables, const int32_t* context_lens, int32_t B, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
    int32_t max_context_len, float scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
    int32_t q_dtype, const int32_t* host_context_lens, pkv_stream_t stream) {
  return fp8_partitions("paged_attention_decode_fp8_partitions", out, out_dtype, query, k_cache, v_cache, k_scale,
                        v_scale, block_tables, context_lens, B, num_q_heads, num_kv_heads, head_dim, block_size,
                        max_blocks_per_seq, num_blocks, max_context_len, scale, partition_size, workspace,
                        workspace_bytes, q_dtype, host_context_lens, stream);
}

extern "C" int paged_attention_decode_fp8(void* out, int32_t out_dtype, const void* query, const void* k_cache,
                                          const void* v_cache, const void* k_scale, const void* v_scale,
                                          const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                          int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                                          int32_t max_context_len, float scale, int32_t partition_size,
                                          void* workspace, size_t workspace_bytes, int32_t q_dtype,
                                          const int32_t* host_context_lens, pkv_stream_t stream) {
  int st = paged_attention_decode_fp8_partitions(out, out_dtype, query, k_cache, v_cache, k_scale, v_scale,
                                                 block_tables, context_lens, B, num_q_heads, num_kv_heads, head_dim,
                                                 block_size, max_blocks_per_seq, num_blocks, max_context_len, scale,
                                                 partition_size, workspace, workspace_bytes, q_dtype,
                                                 host_context_lens, stream);
  if (st != PKV_OK) return st;
  return paged_attention_decode_reduce(out, out_dtype, context_lens, B, num_q_heads, head_dim, max_context_len,
                                       partition_size, workspace, workspace_bytes, stream);
}

extern "C" int paged_attention_decode_append_fp8(void* out, int32_t out_dtype, const void* query, const void* new_key,
                                                 const void* new_value, void* k_cache, void* v_cache, void* k_scale,
                                                 void* v_scale, const int32_t* block_tables,
                                                 const int32_t* context_lens, int32_t B, int32_t num_q_heads,
                                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                                 int32_t max_blocks_per_seq, int32_t num_blocks,
                                                 int32_t max_context_len, float scale, int32_t partition_size,
                                                 void* workspace, size_t workspace_bytes, int32_t q_dtype,
                                                 const int32_t* host_context_lens, pkv_stream_t stream) {
  int st = fp8_partitions("paged_attention_decode_append_fp8", out, out_dtype, query, k_cache, v_cache, k_scale,
                          v_scale, block_tables, context_lens, B, num_q_heads, num_kv_heads, head_dim, block_size,
                          max_blocks_per_seq, num_blocks, max_context_len, scale, partition_size, workspace,
                          workspace_bytes, q_dtype, host_context_lens, stream, new_key, new_value);
  if (st != PKV_OK) return st;
  return paged_attention_decode_reduce(out, out_dtype, context_lens, B, num_q_heads, head_dim, max_context_len,
                                       partition_size, workspace, workspace_bytes, stream);
}

extern "C" int paged_attention_decode_grouped_fp8(void* out, int32_t out_dtype, const void* query, const void* k_cache,
                                                  const void* v_cache, const void* k_scale, const void* v_scale,
                                                  const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                                                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                                  int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                                                  int32_t max_context_len, float scale, int32_t partition_size,
                                                  void* workspace, size_t workspace_bytes, int32_t q_dtype,
                                                  int32_t group_size, pkv_stream_t stream) {
  const char* fn = "paged_attention_decode_grouped_fp8";
  if (group_size < 1) return fail(PKV_EINVAL, "%s: group_size %d", fn, group_size);
  if (group_size == 1)
    return paged_attention_decode_fp8(out, out_dtype, query, k_cache, v_cache, k_scale, v_scale, block_tables,
                                      context_lens, B, num_q_heads, num_kv_heads, head_dim, block_size,
                                      max_blocks_per_seq, num_blocks, max_context_len, scale, partition_size,
                                      workspace, workspace_bytes, q_dtype, nullptr, stream);
  Fp8Args a;
  bool wide = false, empty = true;
  int st = fp8_setup(fn, a, wide, empty, out, out_dtype, query, k_cache, v_cache, k_scale, v_scale, block_tables,
                     context_lens, B, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                     max_context_len, scale, partition_size, workspace, workspace_bytes, q_dtype, nullptr, nullptr,
                     nullptr);
  if (st != PKV_OK) return st;
  const int G = num_q_heads / num_kv_heads;
  const int cols = group_size * G;
  if (cols != 8 && cols != 16)
    return fail(PKV_EUNSUPPORTED, "%s: group_size x (num_q_heads / num_kv_heads) = %d, must be 8 or 16", fn, cols);
  if (empty) return PKV_OK;
  const int ngroups = (B + group_size - 1) / group_size;
  hipStream_t s = as_stream(stream);
  const bool f32out = out_dtype == PKV_F32;
  bool ok;
  if (q_dtype == PKV_BF16)
    ok = f32out ? launch_fp8_group_dim<PKV_BF16, PKV_F32>(a, B, head_dim, G, group_size, ngroups, wide, s)
                : launch_fp8_group_dim<PKV_BF16, PKV_BF16>(a, B, head_dim, G, group_size, ngroups, wide, s);
  else
    ok = f32out ? launch_fp8_group_dim<PKV_F16, PKV_F32>(a, B, head_dim, G, group_size, ngroups, wide, s)
                : launch_fp8_group_dim<PKV_F16, PKV_F16>(a, B, head_dim, G, group_size, ngroups, wide, s);
  if (!ok) return fail(PKV_EUNSUPPORTED, "%s: group_size %d with group %d", fn, group_size, G);
  st = check_launch(fn);
  if (st != PKV_OK) return st;
  return paged_attention_decode_reduce(out, out_dtype, context_lens, B, num_q_heads, head_dim, max_context_len,
                                       partition_size, workspace, workspace_bytes, stream);
}
