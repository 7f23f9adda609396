// One workgroup of chunked-prefill causal attention against the paged cache, shared by the
// prefill kernel (csrc/prefill.hip) and the mixed decode + prefill launch (csrc/mixed.hip).  What
// is computed and how it maps onto the MI355X is described at the top of csrc/prefill.hip.
#pragma once
#include <type_traits>

#include "fp8_device.h"

namespace pkv {
namespace {

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
  const float* ksc;  // fp8 cache only: K / V scales, fp32 [num_blocks][Hkv][16]
  const float* vsc;
};

// One workgroup = 16 chunk rows x the G query heads of one KV head.  A wave owns HPW = min(G, 2)
// heads of the group (HSETS = G / HPW head sets) over one key split (KSPLIT splits of the row
// tile's keys; HSETS x KSPLIT = 8 waves, two per SIMD): every K/V fragment it loads feeds the
// Q.K and P.V products of both its heads, halving the vector-memory bytes per matrix
// instruction (more heads per wave overflow the 256 architectural registers).  Each wave walks its consecutive 32-key steps with one step of
// K/V in flight (next K once this step's Q.K products have consumed the K registers, next V
// after the last P.V); block ids of 64 blocks at a time sit one per lane.  The splits are
// merged exactly through LDS (log-sum-exp) at the end.
template <int G>
struct PrefillShape {
  static constexpr int HPW = G < 2 ? G : 2;
  static constexpr int HSETS = G / HPW;
  static constexpr int KSPLIT = 8 / HSETS;
  static constexpr int NWAVES = HSETS * KSPLIT;
};

// LDS of one workgroup of the body below, in floats: the key splits' partial outputs, maxima, sums.
template <int D, int G>
constexpr int prefill_smem_floats() {
  return PrefillShape<G>::KSPLIT * G * 16 * (D + 2);
}

// The body of one workgroup; id = its index among the row_tiles * Hkv workgroups of the chunk.
// smem: prefill_smem_floats<D, G>() floats of LDS.
//
// FP8: the cache holds E4M3 codes with one K and one V scale per (block, head, slot), the query
// and the products are DT (bf16 / fp16).  A lane's 16-byte K load holds dimensions
// [64p + 16 q4, +16) of one token (one 512-byte run per block and 64 dimensions), widened exactly
// into k-steps 2p and 2p + 1; the query fragments take the same dimension order.  A V load is the
// 8 codes of a dimension for the lane's 8 keys ([D][16] tile).  The scales enter outside the
// products: a score is multiplied by its key's scale, a weight by its value's scale before P.V
// (the softmax sum takes the unscaled weight).
template <int DT, int DT_OUT, int D, int G, bool FP8 = false>
__device__ __forceinline__ void prefill_tile(const PrefillArgs& a, int id, float* smem) {
  constexpr int KS = D / 32;
  constexpr int KP = D / 64;  // FP8: 16-byte K loads per token set
  constexpr int NB = D / 16;
  constexpr int TILE = kBlock * D;  // elements (bytes for FP8) of one (block, head) tile
  constexpr int HPW = PrefillShape<G>::HPW;
  constexpr int HSETS = PrefillShape<G>::HSETS;
  constexpr int KSPLIT = PrefillShape<G>::KSPLIT;
  constexpr int NT = PrefillShape<G>::NWAVES * 64;
  constexpr int kTableSteps = 32;

  // XCD-aware order: hardware places workgroup id on XCD (id % 8); give every XCD whole KV heads.
  const int nwg = a.row_tiles * a.Hkv;
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
  const uint8_t* __restrict__ k8 = static_cast<const uint8_t*>(a.k);
  const uint8_t* __restrict__ v8 = static_cast<const uint8_t*>(a.v);

  u32x4 qf[HPW][KS];
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    const uint16_t* qrow =
        static_cast<const uint16_t*>(a.q) + (static_cast<int64_t>(min(my_row, a.C - 1)) * a.Hq + hq0 + h) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      // FP8: k-step 2p + f holds dimensions [64p + 16 q4 + 8f, +8), the K loads' order
      const int d0 = FP8 ? (ks >> 1) * 64 + q4 * 16 + (ks & 1) * 8 : ks * 32 + q4 * 8;
      qf[h][ks] = row_ok ? *reinterpret_cast<const u32x4*>(qrow + d0) : u32x4{0, 0, 0, 0};
    }
  }

  // Q.K product #s row m holds token 8*(m/4) + m%4 + 4s of the step's block m/8; in the K tile
  // order those rows of one k-step are one 512-byte run per block (see k_chunk_pos).  Lane
  // (row, q4) then holds the scores of step keys 8*q4 .. 8*q4+7, the k-range of its P row.
  const bool k_from_b = n16 >= 8;
  const int k_in_tile = FP8 ? (n16 & 7) * 64 + q4 * 16 : (q4 * 8 + (n16 & 7)) * 8;
  const bool v_from_b = q4 >= 2;  // also the block of the lane's 8 keys' scales
  // V tile [token half][D][8 tokens]; FP8: [D][16] codes
  const int v_in_tile = FP8 ? n16 * kBlock + (q4 & 1) * 8 : (q4 & 1) * D * 8 + n16 * 8;
  const int s_in_head = (q4 & 1) * 8;  // FP8: the lane's 8 keys in their block's scale row

  f32x4 o[HPW][NB];
  float m_run[HPW], l_run[HPW];  // per head: reference maximum (log2 domain) and this lane's sum
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[h][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[h] = kNoMax;
    l_run[h] = 0.f;
  }
  float thr[HPW];  // raw-score rescale threshold per head: (m_run + 2^8) / (scale * log2 e)
#pragma unroll
  for (int h = 0; h < HPW; ++h) thr[h] = (kNoMax + kLazyRescaleLog2) / a.scale_log2;

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
    u32x4 k8f[2 * KP];  // FP8: raw codes, token set s at [s * KP + p]
    u32x2 v8f[NB];
    f32x4 ksf[2], vsf[2];  // FP8: scales of the lane's 8 keys
    auto heads = [&](int st, int64_t& hA, int64_t& hB) {
      const int j = 2 * (st - c0);
      const int bA = __builtin_amdgcn_readlane(tab, j);
      const int bB = __builtin_amdgcn_readlane(tab, min(j + 1, cnb - 1));  // a lone last block pairs with itself
      hA = static_cast<int64_t>(bA) * a.Hkv + g;
      hB = static_cast<int64_t>(bB) * a.Hkv + g;
    };
    auto load_k = [&](int st) {
      int64_t hA, hB;
      heads(st, hA, hB);
      if constexpr (FP8) {
        const uint8_t* kp = k8 + (k_from_b ? hB : hA) * TILE + k_in_tile;
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
#pragma unroll
          for (int pp = 0; pp < KP; ++pp)
            k8f[ss * KP + pp] = *reinterpret_cast<const u32x4*>(kp + (pp * 2 + ss) * 512);
        }
        const float* sp = a.ksc + (v_from_b ? hB : hA) * kBlock + s_in_head;
        ksf[0] = *reinterpret_cast<const f32x4*>(sp);
        ksf[1] = *reinterpret_cast<const f32x4*>(sp + 4);
      } else {
        const uint16_t* kp = kc + (k_from_b ? hB : hA) * TILE + k_in_tile;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          kf[ks] = *reinterpret_cast<const u32x4*>(kp + (2 * ks) * 256);
          kf[KS + ks] = *reinterpret_cast<const u32x4*>(kp + (2 * ks + 1) * 256);
        }
      }
    };
    auto load_v = [&](int st) {
      int64_t hA, hB;
      heads(st, hA, hB);
      if constexpr (FP8) {
        const uint8_t* vp = v8 + (v_from_b ? hB : hA) * TILE + v_in_tile;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) v8f[nb] = *reinterpret_cast<const u32x2*>(vp + nb * 16 * kBlock);
        const float* sp = a.vsc + (v_from_b ? hB : hA) * kBlock + s_in_head;
        vsf[0] = *reinterpret_cast<const f32x4*>(sp);
        vsf[1] = *reinterpret_cast<const f32x4*>(sp + 4);
      } else {
        const uint16_t* vp = vc + (v_from_b ? hB : hA) * TILE + v_in_tile;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) vf[nb] = *reinterpret_cast<const u32x4*>(vp + nb * 16 * 8);
      }
    };

    // One 32-key step for all HPW heads; with `prefetch` the next step's loads are issued as
    // registers free up (the empty asm statements keep them where they are written).
    auto step = [&](int st, const bool prefetch) {
      const int t0 = st * 32;
      const int nvalid = min(32, nkeys - t0);
      const bool masked = t0 + 32 > full_keys;  // causal limit (and the chunk's end) inside this step
      // K operands: the loaded fragments, or (FP8) the codes widened, after which the code
      // registers take the next step's loads.
      u32x4 kk[2 * KS];
      f32x4 ks_cur[2];
      if constexpr (FP8) {
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
#pragma unroll
          for (int pp = 0; pp < KP; ++pp) {
            const u32x4 r = k8f[ss * KP + pp];
            kk[ss * KS + 2 * pp] = widen8<DT>(r[0], r[1]);
            kk[ss * KS + 2 * pp + 1] = widen8<DT>(r[2], r[3]);
          }
        }
        ks_cur[0] = ksf[0];
        ks_cur[1] = ksf[1];
        if (prefetch) {
          asm volatile("" ::: "memory");
          load_k(st + 1);
          asm volatile("" ::: "memory");
        }
      } else {
#pragma unroll
        for (int i = 0; i < 2 * KS; ++i) kk[i] = kf[i];
      }
      f32x4 s1[HPW], s2[HPW];
#pragma unroll
      for (int h = 0; h < HPW; ++h) {
        s1[h] = f32x4{0.f, 0.f, 0.f, 0.f};
        s2[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          s1[h] = mfma16x16x32<DT>(kk[ks], qf[h][ks], s1[h]);
          s2[h] = mfma16x16x32<DT>(kk[KS + ks], qf[h][ks], s2[h]);
        }
      }
      if (!FP8 && prefetch) {
        asm volatile("" ::: "memory");
        load_k(st + 1);
        asm volatile("" ::: "memory");
      }
      if (nvalid < 32) {
        // Keys past the last visible one may be stale (or NaN): zero them in V (FP8: their
        // codes and value scales).
        const int keep = min(8, max(0, nvalid - 8 * q4));
        if constexpr (FP8) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
            for (int wd = 0; wd < 2; ++wd) {
              const int kb = keep - 4 * wd;  // bytes of this dword to keep
              const uint32_t m = kb >= 4 ? 0xFFFFFFFFu : (kb <= 0 ? 0u : (1u << (8 * kb)) - 1u);
              v8f[nb][wd] &= m;
            }
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) vsf[i >> 2][i & 3] = i < keep ? vsf[i >> 2][i & 3] : 0.f;
        } else {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
            for (int wd = 0; wd < 4; ++wd) {
              const uint32_t m = (2 * wd + 1 < keep) ? 0xFFFFFFFFu : ((2 * wd < keep) ? 0x0000FFFFu : 0u);
              vf[nb][wd] &= m;
            }
          }
        }
      }
      // Raw scores; scale * log2(e) > 0 is applied inside the exponent, so maxima of raw scores
      // give the maxima of scaled ones.  Both heads go through each phase before the next one, so
      // that the common path (no mask, no rescale) is one basic block in which the compiler can
      // issue one head's softmax arithmetic between the other head's matrix instructions.
      // FP8: the key's scale (>= 0) is part of the raw score.
      float sc[HPW][8];
#pragma unroll
      for (int h = 0; h < HPW; ++h) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sc[h][j] = FP8 ? s1[h][j] * ks_cur[0][j] : s1[h][j];
          sc[h][4 + j] = FP8 ? s2[h][j] * ks_cur[1][j] : s2[h][j];
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
      // The raw-score threshold thr = (m_run + 2^8) / c saves the scaling of the maxima, and the
      // NaN-propagating maximum needs no canonicalising of the matrix results (v_maximum3).
      // Masked scores are -inf, never NaN, so both maxima agree here.
      float lmax[HPW];
      bool big = false;
#pragma unroll
      for (int h = 0; h < HPW; ++h) {
        lmax[h] = sc[h][0];
#pragma unroll
        for (int i = 1; i < 8; ++i) lmax[h] = __builtin_elementwise_maximum(lmax[h], sc[h][i]);
        big = big || (lmax[h] > thr[h]);
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
          thr[h] = (m_new + kLazyRescaleLog2) / c;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float f = __shfl(alpha, 4 * q4 + j);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) o[h][nb][j] *= f;
          }
        }
      }
      // V operands: the loaded fragments, or (FP8) the codes widened and the value scales kept,
      // after which their registers take the next step's loads.
      u32x4 vv[NB];
      float vs_cur[8];
      if constexpr (FP8) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) vv[nb] = widen8<DT>(v8f[nb][0], v8f[nb][1]);
#pragma unroll
        for (int i = 0; i < 8; ++i) vs_cur[i] = vsf[i >> 2][i & 3];
        if (prefetch) {
          asm volatile("" ::: "memory");
          load_v(st + 1);
          asm volatile("" ::: "memory");
        }
      } else {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) vv[nb] = vf[nb];
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
        if constexpr (FP8) {
#pragma unroll
          for (int i = 0; i < 8; ++i) pv[i] *= vs_cur[i];
        }
        // hi = the weights rounded to 16 bits, lo = the rounding residuals rounded to 16 bits.
        u32x4 hi, lo;
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
          hi[wd] = pack2<DT>(pv[2 * wd], pv[2 * wd + 1]);
          lo[wd] = pack2<DT>(pv[2 * wd] - low_half<DT>(hi[wd]), pv[2 * wd + 1] - high_half<DT>(hi[wd]));
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          o[h][nb] = mfma16x16x32<DT>(hi, vv[nb], o[h][nb]);
          o[h][nb] = mfma16x16x32<DT>(lo, vv[nb], o[h][nb]);
        }
      }
      if (!FP8 && prefetch) {
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
  float (&sO)[KSPLIT][G][16][D] = *reinterpret_cast<float (*)[KSPLIT][G][16][D]>(smem);
  float (&sM)[KSPLIT][G][16] = *reinterpret_cast<float (*)[KSPLIT][G][16]>(smem + KSPLIT * G * 16 * D);
  float (&sL)[KSPLIT][G][16] =
      *reinterpret_cast<float (*)[KSPLIT][G][16]>(smem + KSPLIT * G * 16 * D + KSPLIT * G * 16);
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

}  // namespace
}  // namespace pkv
