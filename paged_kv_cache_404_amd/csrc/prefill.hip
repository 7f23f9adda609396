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
// MI355X mapping: a wavefront owns 16 consecutive chunk rows of one query head; a workgroup holds
// the G query heads of one GQA group (same rows, same K/V tiles, which therefore hit in cache
// after the first wave).  Per 32-token key step, S^T = K.Q^T (2 x D/32 MFMA 16x16x32) and
// O += P.V (D/16 MFMA, twice: P split into hi + lo 16-bit rows so the weights keep ~16 mantissa
// bits).  The causal limit only masks the last steps of each row tile.  Workgroups are ordered
// so that consecutive ids on one XCD work on the same KV head (its K/V then stay in that XCD's L2).
#include <cmath>

#include "device.h"

namespace pkv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyRescaleLog2 = 8.0f;

struct PrefillArgs {
  void* out;
  const void* q;
  const void* k;
  const void* v;
  const int32_t* table;
  int32_t ctx_start;
  int32_t C;
  int32_t Hq;
  int32_t Hkv;
  int32_t num_blocks;
  int32_t row_tiles;  // ceil(C / 16)
  float scale_log2;
};

template <int DT>
__device__ __forceinline__ uint32_t to16(float x) {
  if constexpr (DT == PKV_BF16) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
  } else {
    return __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
  }
}
template <int DT>
__device__ __forceinline__ float from16(uint32_t b) {
  if constexpr (DT == PKV_BF16) {
    return bf16_bits_to_float(b);
  } else {
    return f16_bits_to_float(b);
  }
}
template <int DT>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (DT == PKV_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  }
}

template <int DT, int DT_OUT, int D, int G>
__global__ void __launch_bounds__(G * 64) prefill_mfma_kernel(PrefillArgs a) {
  constexpr int KS = D / 32;
  constexpr int NB = D / 16;
  constexpr int TILE = kBlock * D;

  // XCD-aware order: hardware places workgroup id on XCD (id % 8); give every XCD whole KV heads.
  const int nwg = a.row_tiles * a.Hkv;
  const int id = blockIdx.x;
  int g, tile;
  if (nwg % 8 == 0) {
    const int per_xcd = nwg / 8;
    const int lin = (id % 8) * per_xcd + id / 8;  // consecutive lin share a KV head
    g = lin / a.row_tiles;
    tile = lin % a.row_tiles;
  } else {
    g = id / a.row_tiles;
    tile = id % a.row_tiles;
  }
  // Longest rows first inside a head: later tiles see more keys.
  tile = a.row_tiles - 1 - tile;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;  // query head within the group
  const int hq = g * G + w;
  const int n16 = lane & 15;
  const int q4 = lane >> 4;
  const int i0 = tile * 16;            // first chunk row of this tile
  const int my_row = i0 + n16;         // chunk row held in this lane's S^T column
  const bool row_ok = my_row < a.C;
  const int row_lim = a.ctx_start + min(my_row, a.C - 1);  // last visible key position of that row

  const uint16_t* __restrict__ kc = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ vc = static_cast<const uint16_t*>(a.v);

  u32x4 qf[KS];
  {
    const uint16_t* qrow =
        static_cast<const uint16_t*>(a.q) + (static_cast<int64_t>(min(my_row, a.C - 1)) * a.Hq + hq) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = row_ok ? *reinterpret_cast<const u32x4*>(qrow + ks * 32 + q4 * 8) : u32x4{0, 0, 0, 0};
  }

  // Q.K product #s row m holds token 8*(m/4) + m%4 + 4s of the step's block m/8; in the K tile
  // order those rows of one k-step are one 512-byte run per block (see k_chunk_pos).
  const bool k_from_b = n16 >= 8;
  const int k_in_tile = (q4 * 8 + (n16 & 7)) * 8;
  const int vhalf = q4 >> 1;
  const int vcol = (q4 & 1) * 8;

  f32x4 o[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int last_row = min(i0 + 15, a.C - 1);
  const int nkeys = a.ctx_start + last_row + 1;  // keys any row of the tile can see
  const int full_keys = a.ctx_start + i0 + 1;    // keys every row of the tile sees
  const int nsteps = (nkeys + 31) >> 5;
  for (int st = 0; st < nsteps; ++st) {
    const int t0 = st * 32;
    const int nvalid = min(32, nkeys - t0);
    const int lb = t0 >> 4;
    // block ids are a precondition; clamping turns a bad id into a wrong value instead of a fault
    const int blkA = min(max(a.table[lb], 0), a.num_blocks - 1);
    const int blkB = nvalid > 16 ? min(max(a.table[lb + 1], 0), a.num_blocks - 1) : blkA;
    const int64_t tileA = (static_cast<int64_t>(blkA) * a.Hkv + g) * TILE;
    const int64_t tileB = (static_cast<int64_t>(blkB) * a.Hkv + g) * TILE;

    const uint16_t* kp = kc + (k_from_b ? tileB : tileA) + k_in_tile;
    u32x4 k1[KS], k2[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      k1[ks] = *reinterpret_cast<const u32x4*>(kp + (2 * ks) * 256);
      k2[ks] = *reinterpret_cast<const u32x4*>(kp + (2 * ks + 1) * 256);
    }
    const uint16_t* vbase = vc + (vhalf ? tileB : tileA) + n16 * kBlock + vcol;
    u32x4 vf[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) vf[nb] = *reinterpret_cast<const u32x4*>(vbase + nb * 16 * kBlock);

    f32x4 s1 = {0.f, 0.f, 0.f, 0.f}, s2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s1 = mfma16x16x32<DT>(k1[ks], qf[ks], s1);
      s2 = mfma16x16x32<DT>(k2[ks], qf[ks], s2);
    }
    // Lane (row n16, q4) holds the scores of step tokens 8*q4 + i, i = 0..7.
    const int tb = t0 + 8 * q4;
    const bool masked_step = t0 + 32 > full_keys;
    float sc[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sc[j] = s1[j] * a.scale_log2;
      sc[4 + j] = s2[j] * a.scale_log2;
    }
    if (masked_step) {
#pragma unroll
      for (int i = 0; i < 8; ++i) sc[i] = (row_ok && tb + i <= row_lim) ? sc[i] : -INFINITY;
    }
    float bmax = sc[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) bmax = fmaxf(bmax, sc[i]);
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32));

    const bool need = row_ok && (bmax > m_run + kLazyRescaleLog2);
    if (__any(need)) {
      const float m_new = need ? bmax : m_run;
      const float alpha = need ? fast_exp2(m_run - m_new) : 1.0f;
      l_run *= alpha;
      m_run = m_new;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float f = __shfl(alpha, 4 * q4 + j);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) o[nb][j] *= f;
      }
    }
    float pv[8];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pv[i] = row_ok ? fast_exp2(sc[i] - m_run) : 0.f;
      psum += pv[i];
    }
    l_run += psum;
    u32x4 hi, lo;
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      const uint32_t h0 = to16<DT>(pv[2 * wd]);
      const uint32_t h1 = to16<DT>(pv[2 * wd + 1]);
      hi[wd] = h0 | (h1 << 16);
      lo[wd] = to16<DT>(pv[2 * wd] - from16<DT>(h0)) | (to16<DT>(pv[2 * wd + 1] - from16<DT>(h1)) << 16);
    }
    if (nvalid < 32) {
      // Keys past the last visible one may be stale (or NaN): zero them in V.
      const int keep = min(8, max(0, nvalid - 8 * q4));
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
          const uint32_t m = (2 * wd + 1 < keep) ? 0xFFFFFFFFu : ((2 * wd < keep) ? 0x0000FFFFu : 0u);
          vf[nb][wd] &= m;
        }
      }
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      o[nb] = mfma16x16x32<DT>(hi, vf[nb], o[nb]);
      o[nb] = mfma16x16x32<DT>(lo, vf[nb], o[nb]);
    }
  }

  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  // O row r = 4*q4 + j is chunk row i0 + r; column nb*16 + n16.
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 4 * q4 + j;
    const float lr = __shfl(l_run, r);
    const int row = i0 + r;
    if (row < a.C) {
      const float inv = 1.0f / lr;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        store_from_float<DT_OUT>(a.out, (static_cast<int64_t>(row) * a.Hq + hq) * D + nb * 16 + n16, o[nb][j] * inv);
    }
  }
}

template <int DT, int DT_OUT, int D>
void launch_g(const PrefillArgs& a, hipStream_t s) {
  const dim3 grid(a.row_tiles * a.Hkv);
  switch (a.Hq / a.Hkv) {
    case 1: hipLaunchKernelGGL((prefill_mfma_kernel<DT, DT_OUT, D, 1>), grid, dim3(64), 0, s, a); break;
    case 2: hipLaunchKernelGGL((prefill_mfma_kernel<DT, DT_OUT, D, 2>), grid, dim3(128), 0, s, a); break;
    case 4: hipLaunchKernelGGL((prefill_mfma_kernel<DT, DT_OUT, D, 4>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((prefill_mfma_kernel<DT, DT_OUT, D, 8>), grid, dim3(512), 0, s, a); break;
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
  if (dtype == PKV_F32) return fail(PKV_EUNSUPPORTED, "%s: fp32 caches are not implemented (bf16 or fp16)", fn);
  if (out_dtype != PKV_F32 && out_dtype != dtype)
    return fail(PKV_EINVAL, "%s: out_dtype must be PKV_F32 or the input dtype", fn);
  if (ctx_start < 0 || C < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 || block_size <= 0)
    return fail(PKV_EINVAL, "%s: bad sizes", fn);
  if (num_q_heads % num_kv_heads != 0) return fail(PKV_EINVAL, "%s: num_q_heads not a multiple of num_kv_heads", fn);
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
  if (dtype == PKV_BF16) {
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
