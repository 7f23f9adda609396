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
// MI355X mapping: a workgroup owns 16 consecutive chunk rows of the G query heads of one KV
// head; its waves split the key range and the heads, and each wave serves two heads from every
// K/V fragment it loads.  Per
// 32-key step, S^T = K.Q^T (2 x D/32 MFMA 16x16x32) and O += P.V (D/16 MFMA, twice: P split
// into hi + lo 16-bit rows so the weights keep ~16 mantissa bits).  The causal limit only masks
// the last steps of each row tile.  Workgroups are ordered so that consecutive ids on one XCD
// work on the same KV head (its K/V then stay in that XCD's L2).
#include <cmath>

#include "device.h"

namespace pkv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyRescaleLog2 = 8.0f;
// Running maximum before any visible key: finite, so exp2(x - m) needs no -inf guard, and far
// below any score (a split that sees no key of a row keeps it; the merge weighs it exp2(-1e30) = 0).
constexpr float kNoMax = -1e30f;

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
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (DT == PKV_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  }
}

// One workgroup = 16 chunk rows x the G query heads of one KV head.  A wave owns HPW = min(G, 2)
// heads of the group (HSETS = G / HPW head sets) over one key split (KSPLIT splits of the row
// tile's keys; HSETS x KSPLIT <= 8 waves, two per SIMD): every K/V fragment it loads feeds the
// Q.K and P.V products of both its heads, halving the vector-memory bytes per matrix
// instruction (more heads per wave overflow the 256 architectural registers).  Each wave walks its consecutive 32-key steps with one step of
// K/V in flight (next K once this step's Q.K products have consumed the K registers, next V
// after the last P.V); block ids of 64 blocks at a time sit one per lane.  The splits are
// merged exactly through LDS (log-sum-exp) at the end.
template <int G>
struct PrefillShape {
  static constexpr int HPW = G < 2 ? G : 2;
  static constexpr int HSETS = G / HPW;
  static constexpr int KSPLIT = HSETS >= 4 ? 2 : 4;
  static constexpr int NWAVES = HSETS * KSPLIT;
};

template <int DT, int DT_OUT, int D, int G>
__global__ void __launch_bounds__(PrefillShape<G>::NWAVES * 64) prefill_mfma_kernel(PrefillArgs a) {
  constexpr int KS = D / 32;
  constexpr int NB = D / 16;
  constexpr int TILE = kBlock * D;
  constexpr int HPW = PrefillShape<G>::HPW;
  constexpr int HSETS = PrefillShape<G>::HSETS;
  constexpr int KSPLIT = PrefillShape<G>::KSPLIT;
  constexpr int NT = PrefillShape<G>::NWAVES * 64;
  constexpr int kTableSteps = 32;

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
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hs = w % HSETS;  // head set
  const int sp = w / HSETS;  // key split
  const int hq0 = g * G + hs * HPW;
  const int n16 = lane & 15;
  const int q4 = lane >> 4;
  const int i0 = tile * 16;       // first chunk row of this tile
  const int my_row = i0 + n16;    // chunk row held in this lane's S^T column
  const bool row_ok = my_row < a.C;
  const int row_lim = a.ctx_start + min(my_row, a.C - 1);  // last visible key position of that row

  const uint16_t* __restrict__ kc = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ vc = static_cast<const uint16_t*>(a.v);

  u32x4 qf[HPW][KS];
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    const uint16_t* qrow =
        static_cast<const uint16_t*>(a.q) + (static_cast<int64_t>(min(my_row, a.C - 1)) * a.Hq + hq0 + h) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[h][ks] = row_ok ? *reinterpret_cast<const u32x4*>(qrow + ks * 32 + q4 * 8) : u32x4{0, 0, 0, 0};
  }

  // Q.K product #s row m holds token 8*(m/4) + m%4 + 4s of the step's block m/8; in the K tile
  // order those rows of one k-step are one 512-byte run per block (see k_chunk_pos).  Lane
  // (row, q4) then holds the scores of step keys 8*q4 .. 8*q4+7, the k-range of its P row.
  const bool k_from_b = n16 >= 8;
  const int k_in_tile = (q4 * 8 + (n16 & 7)) * 8;
  const bool v_from_b = q4 >= 2;
  const int v_in_tile = n16 * kBlock + (q4 & 1) * 8;

  f32x4 o[HPW][NB];
  float m_run[HPW], l_run[HPW];  // per head: reference maximum (log2 domain) and this lane's sum
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[h][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[h] = kNoMax;
    l_run[h] = 0.f;
  }

  const int last_row = min(i0 + 15, a.C - 1);
  const int nkeys = a.ctx_start + last_row + 1;  // keys any row of the tile can see
  const int full_keys = a.ctx_start + i0 + 1;    // keys every row of the tile sees
  const int nsteps = (nkeys + 31) >> 5;
  const int per_split = (nsteps + KSPLIT - 1) / KSPLIT;
  const int s_lo = min(nsteps, sp * per_split);
  const int s_hi = min(nsteps, s_lo + per_split);
  const int kblocks = (nkeys + 15) >> 4;  // blocks the tile reads; the table holds at least these
  const float c = a.scale_log2;

  for (int c0 = s_lo; c0 < s_hi; c0 += kTableSteps) {
    const int cend = min(s_hi, c0 + kTableSteps);
    const int cb0 = 2 * c0;
    const int cnb = min(2 * kTableSteps, kblocks - cb0);
    // block ids are a precondition; clamping turns a bad id into a wrong value instead of a fault
    const int tab = min(max(a.table[min(cb0 + lane, kblocks - 1)], 0), a.num_blocks - 1);

    u32x4 kf[2 * KS], vf[NB];
    auto tiles = [&](int st, int64_t& tA, int64_t& tB) {
      const int j = 2 * (st - c0);
      const int bA = __builtin_amdgcn_readlane(tab, j);
      const int bB = __builtin_amdgcn_readlane(tab, min(j + 1, cnb - 1));  // a lone last block pairs with itself
      tA = (static_cast<int64_t>(bA) * a.Hkv + g) * TILE;
      tB = (static_cast<int64_t>(bB) * a.Hkv + g) * TILE;
    };
    auto load_k = [&](int st) {
      int64_t tA, tB;
      tiles(st, tA, tB);
      const uint16_t* kp = kc + (k_from_b ? tB : tA) + k_in_tile;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        kf[ks] = *reinterpret_cast<const u32x4*>(kp + (2 * ks) * 256);
        kf[KS + ks] = *reinterpret_cast<const u32x4*>(kp + (2 * ks + 1) * 256);
      }
    };
    auto load_v = [&](int st) {
      int64_t tA, tB;
      tiles(st, tA, tB);
      const uint16_t* vp = vc + (v_from_b ? tB : tA) + v_in_tile;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) vf[nb] = *reinterpret_cast<const u32x4*>(vp + nb * 16 * kBlock);
    };

    // One 32-key step for all HPW heads; with `prefetch` the next step's loads are issued as
    // registers free up (the empty asm statements keep them where they are written).
    auto step = [&](int st, const bool prefetch) {
      const int t0 = st * 32;
      const int nvalid = min(32, nkeys - t0);
      const bool masked = t0 + 32 > full_keys;  // causal limit (and the chunk's end) inside this step
      f32x4 s1[HPW], s2[HPW];
#pragma unroll
      for (int h = 0; h < HPW; ++h) {
        s1[h] = f32x4{0.f, 0.f, 0.f, 0.f};
        s2[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          s1[h] = mfma16x16x32<DT>(kf[ks], qf[h][ks], s1[h]);
          s2[h] = mfma16x16x32<DT>(kf[KS + ks], qf[h][ks], s2[h]);
        }
      }
      if (prefetch) {
        asm volatile("" ::: "memory");
        load_k(st + 1);
        asm volatile("" ::: "memory");
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
      // Raw scores; scale * log2(e) > 0 is applied inside the exponent, so maxima of raw scores
      // give the maxima of scaled ones.  Both heads go through each phase before the next one, so
      // that the common path (no mask, no rescale) is one basic block in which the compiler can
      // issue one head's softmax arithmetic between the other head's matrix instructions.
      float sc[HPW][8];
#pragma unroll
      for (int h = 0; h < HPW; ++h) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sc[h][j] = s1[h][j];
          sc[h][4 + j] = s2[h][j];
        }
      }
      if (masked) {
        // Keys visible to this lane's row in this step: t0 + 8*q4 + i <= row_lim.  The empty asm
        // keeps the compares inside the (rarely taken) branch.
        int lim = row_ok ? row_lim - (t0 + 8 * q4) : -1;
        asm volatile("" : "+v"(lim));
#pragma unroll
        for (int h = 0; h < HPW; ++h) {
#pragma unroll
          for (int i = 0; i < 8; ++i) sc[h][i] = (i <= lim) ? sc[h][i] : -INFINITY;
        }
      }
      // Lazy rescale: a row's reference maximum moves only when one of its scores exceeds it by
      // more than 2^8.  Each lane tests its own 8 scores per head; the row maximum over the
      // row's four lanes is formed only when some lane of the wave passes that test.
      float lmax[HPW];
      bool big = false;
#pragma unroll
      for (int h = 0; h < HPW; ++h) {
        lmax[h] = sc[h][0];
#pragma unroll
        for (int i = 1; i < 8; ++i) lmax[h] = fmaxf(lmax[h], sc[h][i]);
        big = big || (lmax[h] * c > m_run[h] + kLazyRescaleLog2);
      }
      if (__any(big)) {
#pragma unroll
        for (int h = 0; h < HPW; ++h) {
          const float bmax = group4_max(lmax[h]) * c;
          const bool need = row_ok && (bmax > m_run[h] + kLazyRescaleLog2);
          const float m_new = need ? bmax : m_run[h];
          const float alpha = need ? fast_exp2(m_run[h] - m_new) : 1.0f;
          l_run[h] *= alpha;
          m_run[h] = m_new;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float f = __shfl(alpha, 4 * q4 + j);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) o[h][nb][j] *= f;
          }
        }
      }
#pragma unroll
      for (int h = 0; h < HPW; ++h) {
        // Before a row's first visible key m_run is the finite kNoMax: masked scores (-inf) get
        // weight exp2(-inf) = 0, and the first real maximum rescales by exp2(kNoMax - m) = 0.
        float pv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) pv[i] = fast_exp2(fmaf(sc[h][i], c, -m_run[h]));
        float psum = pv[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) psum += pv[i];
        l_run[h] += psum;
        // hi = the weights rounded to 16 bits, lo = the rounding residuals rounded to 16 bits.
        u32x4 hi, lo;
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
          hi[wd] = pack2<DT>(pv[2 * wd], pv[2 * wd + 1]);
          lo[wd] = pack2<DT>(pv[2 * wd] - low_half<DT>(hi[wd]), pv[2 * wd + 1] - high_half<DT>(hi[wd]));
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          o[h][nb] = mfma16x16x32<DT>(hi, vf[nb], o[h][nb]);
          o[h][nb] = mfma16x16x32<DT>(lo, vf[nb], o[h][nb]);
        }
      }
      if (prefetch) {
        asm volatile("" ::: "memory");
        load_v(st + 1);
        asm volatile("" ::: "memory");
      }
    };

    int st = c0;
    load_k(st);
    load_v(st);
    for (; st + 1 < cend; ++st) step(st, true);
    step(st, false);
  }

  // Merge the key splits: O row r = 4*q4 + j is chunk row i0 + r, column nb*16 + n16.  Rows of
  // rows past the chunk (row_ok false) hold garbage and are never stored.
  __shared__ float sO[KSPLIT][G][16][D];
  __shared__ float sM[KSPLIT][G][16];
  __shared__ float sL[KSPLIT][G][16];
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    const float l = group4_sum(l_run[h]);
    const int hg = hs * HPW + h;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) sO[sp][hg][4 * q4 + j][nb * 16 + n16] = o[h][nb][j];
    }
    if (q4 == 0) {
      sM[sp][hg][n16] = m_run[h];
      sL[sp][hg][n16] = l;
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * 16 * D; idx += NT) {
    const int h = idx / (16 * D);
    const int r = (idx / D) % 16;
    const int d = idx % D;
    const int row = i0 + r;
    if (row >= a.C) continue;
    float M = sM[0][h][r];
#pragma unroll
    for (int k = 1; k < KSPLIT; ++k) M = fmaxf(M, sM[k][h][r]);
    float acc = 0.f, lsum = 0.f;
#pragma unroll
    for (int k = 0; k < KSPLIT; ++k) {
      const float f = fast_exp2(sM[k][h][r] - M);  // a split that saw no key of the row holds kNoMax -> 0
      acc += f * sO[k][h][r][d];
      lsum += f * sL[k][h][r];
    }
    store_from_float<DT_OUT>(a.out, (static_cast<int64_t>(row) * a.Hq + g * G + h) * D + d, acc / lsum);
  }
}

template <int DT, int DT_OUT, int D, int G>
void launch_one(const PrefillArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((prefill_mfma_kernel<DT, DT_OUT, D, G>), dim3(a.row_tiles * a.Hkv),
                     dim3(PrefillShape<G>::NWAVES * 64), 0, s, a);
}

template <int DT, int DT_OUT, int D>
void launch_g(const PrefillArgs& a, hipStream_t s) {
  switch (a.Hq / a.Hkv) {
    case 1: launch_one<DT, DT_OUT, D, 1>(a, s); break;
    case 2: launch_one<DT, DT_OUT, D, 2>(a, s); break;
    case 4: launch_one<DT, DT_OUT, D, 4>(a, s); break;
    default: launch_one<DT, DT_OUT, D, 8>(a, s); break;
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
