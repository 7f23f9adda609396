// One workgroup of paged decode attention over the FP8 (E4M3) cache, shared by the FP8 decode
// kernels (csrc/fp8.hip) and the mixed decode + prefill launch over that cache (csrc/mixed_fp8.hip).
// The format, layout and what is computed are described at the top of csrc/fp8.hip.
#pragma once
#include <algorithm>
#include <cmath>

#include "fp8_device.h"

namespace pkv {
namespace {

constexpr float kE4M3Max = 448.0f;
constexpr float kLog2eF8 = 1.4426950408889634f;
constexpr float kLazyRescaleLog2F8 = 8.0f;
constexpr int kMaxOrderF8 = 512;

// Four fp32 values -> four E4M3 codes in one dword (byte i = value i), round to nearest even.
__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

struct Fp8Args {
  void* out;
  const void* q;
  const uint8_t* k;
  const uint8_t* v;
  const float* ksc;
  const float* vsc;
  const int32_t* tables;
  const int32_t* lens;
  float* part_ml;
  float* part_o;
  int32_t Hq;
  int32_t Hkv;
  int32_t max_blocks;
  int32_t num_blocks;
  int32_t max_parts;
  int32_t part_size;
  float scale_log2;
  const void* new_k;  // fused append: [B][Hkv][D] of the query's type, the token at position L - 1
  const void* new_v;
  uint8_t* k_out;     // fused append: the caches and scales, written at that token's slot
  uint8_t* v_out;
  float* ksc_out;
  float* vsc_out;
  int32_t num_order;
  int32_t order[kMaxOrderF8];
};

template <int DT>
__device__ __forceinline__ f32x4 mfma_f8(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (DT == PKV_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  }
}

__device__ __forceinline__ int clamp_len_f8(const Fp8Args& a, int b) {
  return min(a.lens[b], min(a.max_parts * a.part_size, a.max_blocks * kBlock));
}
__device__ __forceinline__ int clamp_blk_f8(const Fp8Args& a, int blk) { return min(max(blk, 0), a.num_blocks - 1); }

template <int DT_OUT>
__device__ __forceinline__ void emit_f8(const Fp8Args& a, int b, int hq, int p, int nparts, int d, int D, float m,
                                        float l, float acc) {
  if (nparts == 1) {
    store_from_float<DT_OUT>(a.out, (static_cast<int64_t>(b) * a.Hq + hq) * D + d, acc / l);
  } else {
    const int64_t row = (static_cast<int64_t>(b) * a.Hq + hq) * a.max_parts + p;
    a.part_o[row * D + d] = acc;
    if (d == 0) {
      a.part_ml[row * 2] = m;
      a.part_ml[row * 2 + 1] = l;
    }
  }
}

// Largest magnitude over the 16 lanes of each 16-lane row (every lane takes part).
__device__ __forceinline__ float row16_max(float x) {
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// LDS of one workgroup of the body below, in floats: the waves' partial outputs, maxima and sums.
template <int D, int G, int NW>
constexpr int fp8_decode_smem_floats() {
  return NW * G * D + 2 * NW * G;
}

// The body of one workgroup: KV head g, batch row yb (the sequence is order[yb] when a work order
// is given), partition p; NW waves per partition, wave w takes steps w, w + NW, ...  smem:
// fp8_decode_smem_floats<D, G, NW>() floats of LDS.
//
// NEWTOK (fused append): the token at position L - 1 is this step's new token; its K/V come from
// the input rows new_k / new_v.  The wave that owns the last step of the sequence's last
// partition quantises them exactly as append_fp8_kernel does (one scale per (token, head):
// amax / 448, codes RNE of x * (448 / amax)), puts the codes and scales into its operand
// registers in place of the slot's stale contents, and stores back whole lines: the half of the
// block's K code tile that holds the token's 4-token set, the whole V code tile and both scale
// rows (every other slot with the bytes it was loaded with).  The last block of a sequence is
// private to it, so no other workgroup touches that block in the launch.
template <int DT, int DT_OUT, int D, int G, int NW, bool NEWTOK>
__device__ __forceinline__ void decode_fp8_part(const Fp8Args& a, const int g, const int yb, const int p,
                                                float* smem) {
  static_assert(D == 64 || D == 128, "head_dim");
  constexpr int KP = D / 64;  // 16-byte K loads per token set (two k-steps each)
  constexpr int KS = D / 32;
  constexpr int NB = D / 16;
  constexpr int TILE = kBlock * D;  // bytes of one (block, head) tile
  constexpr int kTableSteps = 32;

  const int b = a.num_order ? a.order[yb] : yb;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pstart = p * a.part_size;
  const int32_t* __restrict__ table = a.tables + static_cast<int64_t>(b) * a.max_blocks;
  const int tab_first = table[min((pstart >> 4) + lane, a.max_blocks - 1)];
  const int L = clamp_len_f8(a, b);
  if (pstart >= L) return;
  const int pend = min(pstart + a.part_size, L);
  const int nparts = (L + a.part_size - 1) / a.part_size;
  const int n16 = lane & 15;
  const int q4 = lane >> 4;
  const int nsteps = (pend - pstart + 31) >> 5;

  // Fused append: where the new token sits in the operand registers of its step.  K codes: lanes
  // n16 == nk_lane (all q4), token set nk_set; V codes and both scales: lanes q4 == nv_q4, byte /
  // element (L - 1) % 8.  The owner's lanes load the token's input values at kernel start.
  const int last_st = nsteps - 1;
  const bool owner = NEWTOK && p == nparts - 1 && w == last_st % NW;
  const int nu = (L - 1) - (pstart + last_st * 32);  // index of the new token inside its step
  const bool nin_b = (nu >> 4) != 0;                // in the step's second block
  const int ntt = (L - 1) & 15;                     // offset inside its block
  const int nk_lane = (nin_b ? 8 : 0) + (ntt >> 3) * 4 + (ntt & 3);
  const int nk_set = (ntt >> 2) & 1;
  const int nv_q4 = (nin_b ? 2 : 0) + (ntt >> 3);
  u32x4 nk[2 * KP];    // lane (nk_lane, q4): dims [64 pp + 16 q4, +16) as two 8-element pieces
  uint32_t nvx[NB];   // lane (n16, nv_q4): dim 16 nb + n16
#pragma unroll
  for (int i = 0; i < 2 * KP; ++i) nk[i] = u32x4{0, 0, 0, 0};
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) nvx[nb] = 0;
  if (owner) {
    const int64_t row = (static_cast<int64_t>(b) * a.Hkv + g) * D;
    const uint16_t* krow = static_cast<const uint16_t*>(a.new_k) + row;
    const uint16_t* vrow = static_cast<const uint16_t*>(a.new_v) + row;
    if ((lane & 15) == nk_lane) {
#pragma unroll
      for (int pp = 0; pp < KP; ++pp) {
        nk[2 * pp] = *reinterpret_cast<const u32x4*>(krow + 64 * pp + 16 * (lane >> 4));
        nk[2 * pp + 1] = *reinterpret_cast<const u32x4*>(krow + 64 * pp + 16 * (lane >> 4) + 8);
      }
    }
    if ((lane >> 4) == nv_q4) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) nvx[nb] = vrow[nb * 16 + (lane & 15)];
    }
  }

  // Query fragments in the K loads' dimension order: k-step 2p + h holds [64p + 16 q4 + 8h, +8).
  u32x4 qf[KS];
  {
    const uint16_t* qrow =
        static_cast<const uint16_t*>(a.q) + (static_cast<int64_t>(b) * a.Hq + g * G + min(n16, G - 1)) * D;
#pragma unroll
    for (int pp = 0; pp < KP; ++pp) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        qf[2 * pp + hf] =
            (n16 < G) ? *reinterpret_cast<const u32x4*>(qrow + 64 * pp + 16 * q4 + 8 * hf) : u32x4{0, 0, 0, 0};
      }
    }
  }
  // Q.K product #s row m holds token 8*(m/4) + m%4 + 4s of block m/8: lane (m = n16, q4) reads
  // that token's dimensions [64p + 16 q4, +16).  Lane (head n16, q4) then holds the scores of step
  // tokens 8*q4 .. 8*q4+7 (block q4/2, slots 8*(q4%2) ..), whose scales it loads.
  const bool k_from_b = n16 >= 8;
  const int k_in_tile = (n16 & 7) * 64 + q4 * 16;
  const bool v_from_b = q4 >= 2;
  const int v_in_tile = n16 * kBlock + (q4 & 1) * 8;
  const bool s_from_b = q4 >= 2;
  const int s_in_head = (q4 & 1) * 8;

  f32x4 o[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;

  for (int c0 = 0; c0 < nsteps; c0 += kTableSteps) {
    const int cend = min(nsteps, c0 + kTableSteps);
    int st = c0 + w;
    if (st >= cend) continue;
    const int cb0 = (pstart >> 4) + 2 * c0;
    const int cnb = min(2 * kTableSteps, ((pend + 15) >> 4) - cb0);
    const int tab = clamp_blk_f8(a, c0 == 0 ? tab_first : table[min(cb0 + lane, a.max_blocks - 1)]);

    u32x4 kraw[2 * KP];
    u32x2 vraw[NB];
    f32x4 ksc[2], vsc[2];
    auto heads = [&](int s, int64_t& hA, int64_t& hB) {
      const int jj = 2 * (s - c0);
      const int bA = __builtin_amdgcn_readlane(tab, jj);
      const int bB = __builtin_amdgcn_readlane(tab, min(jj + 1, cnb - 1));  // a lone last block pairs with itself
      hA = static_cast<int64_t>(bA) * a.Hkv + g;
      hB = static_cast<int64_t>(bB) * a.Hkv + g;
    };
    auto load_k = [&](int s) {
      int64_t hA, hB;
      heads(s, hA, hB);
      const uint8_t* kp = a.k + (k_from_b ? hB : hA) * TILE + k_in_tile;
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
#pragma unroll
        for (int pp = 0; pp < KP; ++pp)
          kraw[ss * KP + pp] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + (pp * 2 + ss) * 512));
      }
    };
    auto load_ks = [&](int s) {
      int64_t hA, hB;
      heads(s, hA, hB);
      const float* sp = a.ksc + (s_from_b ? hB : hA) * kBlock + s_in_head;
      ksc[0] = *reinterpret_cast<const f32x4*>(sp);
      ksc[1] = *reinterpret_cast<const f32x4*>(sp + 4);
    };
    auto load_v = [&](int s) {
      int64_t hA, hB;
      heads(s, hA, hB);
      const uint8_t* vp = a.v + (v_from_b ? hB : hA) * TILE + v_in_tile;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        vraw[nb] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(vp + nb * 16 * kBlock));
    };
    auto load_vs = [&](int s) {
      int64_t hA, hB;
      heads(s, hA, hB);
      const float* sp = a.vsc + (s_from_b ? hB : hA) * kBlock + s_in_head;
      vsc[0] = *reinterpret_cast<const f32x4*>(sp);
      vsc[1] = *reinterpret_cast<const f32x4*>(sp + 4);
    };

    auto step = [&](int s, const bool prefetch) {
      const int nvalid = min(32, pend - (pstart + s * 32));
      if (!prefetch && owner && s == last_st) {
        // The owner's last step (never issued with a successor) holds the new token's block.
        // The asm operands keep the compiler from waiting for the token's loads any earlier.
#pragma unroll
        for (int i = 0; i < 2 * KP; ++i) asm volatile("" : "+v"(nk[i]));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) asm volatile("" : "+v"(nvx[nb]));
        // K: amax over the token's D values (4 lanes x 16 KP), then codes of x * (448 / amax).
        float kx[2 * KP][8];
        float ka = 0.f;
#pragma unroll
        for (int i = 0; i < 2 * KP; ++i) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t bits = (nk[i][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
            kx[i][e] = DT == PKV_BF16 ? bf16_bits_to_float(bits) : f16_bits_to_float(bits);
            ka = fmaxf(ka, fabsf(kx[i][e]));
          }
        }
        // Full over the token's 4 lanes, then from its lane to all (the scale goes to lanes of
        // every row: those of the q4 group that holds the token's scores).
        ka = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, group4_max(ka)), nk_lane));
        const float kscale = __fdiv_rn(ka, kE4M3Max);
        const float kinv = ka > 0.f ? __fdiv_rn(kE4M3Max, ka) : 0.f;
        // V: amax over the token's D values (16 lanes x NB).
        float vx[NB];
        float va = 0.f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          vx[nb] = DT == PKV_BF16 ? bf16_bits_to_float(nvx[nb]) : f16_bits_to_float(nvx[nb]);
          va = fmaxf(va, fabsf(vx[nb]));
        }
        va = row16_max(va);  // full in the lanes q4 == nv_q4, the only ones that use it
        const float vscale = __fdiv_rn(va, kE4M3Max);
        const float vinv = va > 0.f ? __fdiv_rn(kE4M3Max, va) : 0.f;
        if ((lane & 15) == nk_lane) {
#pragma unroll
          for (int pp = 0; pp < KP; ++pp) {
            u32x4 c;
#pragma unroll
            for (int wd = 0; wd < 4; ++wd) {
              const float* x = &kx[2 * pp + (wd >> 1)][4 * (wd & 1)];
              c[wd] = pack4_fp8(x[0] * kinv, x[1] * kinv, x[2] * kinv, x[3] * kinv);
            }
            if (nk_set)
              kraw[KP + pp] = c;
            else
              kraw[pp] = c;
          }
        }
        if (q4 == nv_q4) {
          const int e = ntt & 7;
          const uint32_t sh = 8 * (e & 3);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const uint32_t code = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(vx[nb] * vinv, 0.f, 0, false)) &
                                  0xFFu;
#pragma unroll
            for (int wd = 0; wd < 2; ++wd) {
              if (wd == (e >> 2)) vraw[nb][wd] = (vraw[nb][wd] & ~(0xFFu << sh)) | (code << sh);
            }
          }
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            if (jj == e) {
              ksc[jj >> 2][jj & 3] = kscale;
              vsc[jj >> 2][jj & 3] = vscale;
            }
          }
        }
        // Store back, with the loads' own lane patterns (every line written whole): the half of
        // the K code tile that holds the token's 4-token set (its codes lie nowhere else), the
        // whole V code tile (the token has a byte in every line of it) and both scale rows.
        int64_t hA, hB;
        heads(s, hA, hB);
        const int64_t hN = nin_b ? hB : hA;
        if (k_from_b == nin_b) {
          uint8_t* kp = a.k_out + hN * TILE + k_in_tile + nk_set * 512;
#pragma unroll
          for (int pp = 0; pp < KP; ++pp)
            *reinterpret_cast<u32x4*>(kp + pp * 2 * 512) = nk_set ? kraw[KP + pp] : kraw[pp];
        }
        if (v_from_b == nin_b) {
          uint8_t* vp = a.v_out + hN * TILE + v_in_tile;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) *reinterpret_cast<u32x2*>(vp + nb * 16 * kBlock) = vraw[nb];
        }
        if (s_from_b == nin_b && n16 == 0) {
          float* kso = a.ksc_out + hN * kBlock + s_in_head;
          float* vso = a.vsc_out + hN * kBlock + s_in_head;
          *reinterpret_cast<f32x4*>(kso) = ksc[0];
          *reinterpret_cast<f32x4*>(kso + 4) = ksc[1];
          *reinterpret_cast<f32x4*>(vso) = vsc[0];
          *reinterpret_cast<f32x4*>(vso + 4) = vsc[1];
        }
      }
      // Widen this step's K codes; the K registers are then free for the next step's loads.
      u32x4 kf[2][KS];
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
#pragma unroll
        for (int pp = 0; pp < KP; ++pp) {
          const u32x4 r = kraw[ss * KP + pp];
          kf[ss][2 * pp] = widen8<DT>(r[0], r[1]);
          kf[ss][2 * pp + 1] = widen8<DT>(r[2], r[3]);
        }
      }
      if (prefetch) {
        asm volatile("" ::: "memory");
        load_k(s + NW);
        asm volatile("" ::: "memory");
      }
      f32x4 s1 = {0.f, 0.f, 0.f, 0.f}, s2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s1 = mfma_f8<DT>(kf[0][ks], qf[ks], s1);
        s2 = mfma_f8<DT>(kf[1][ks], qf[ks], s2);
      }
      const int tb = 8 * q4;
      float sc[8];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        sc[jj] = (n16 < G && tb + jj < nvalid) ? s1[jj] * (ksc[0][jj] * a.scale_log2) : -INFINITY;
        sc[4 + jj] = (n16 < G && tb + 4 + jj < nvalid) ? s2[jj] * (ksc[1][jj] * a.scale_log2) : -INFINITY;
      }
      if (prefetch) load_ks(s + NW);
      float bmax = sc[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) bmax = fmaxf(bmax, sc[i]);
      bmax = group4_max(bmax);
      const bool need = (n16 < G) && (bmax > m_run + kLazyRescaleLog2F8);
      if (__any(need)) {
        const float m_new = need ? bmax : m_run;
        const float alpha = need ? fast_exp2(m_run - m_new) : 1.0f;
        l_run *= alpha;
        m_run = m_new;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float f = __shfl(alpha, (4 * q4 + jj) % G);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) o[nb][jj] *= f;
        }
      }
      float pw[8];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float pv = (n16 < G) ? fast_exp2(sc[i] - m_run) : 0.f;
        psum += pv;
        // the value scale of a token past the context may be stale (NaN): its weight is 0 anyway
        const float vs = tb + i < nvalid ? vsc[i >> 2][i & 3] : 0.f;
        pw[i] = pv * vs;
      }
      l_run += psum;
      if (prefetch) load_vs(s + NW);
      u32x4 hi, lo;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        hi[wd] = pack2<DT>(pw[2 * wd], pw[2 * wd + 1]);
        lo[wd] = pack2<DT>(pw[2 * wd] - low_half<DT>(hi[wd]), pw[2 * wd + 1] - high_half<DT>(hi[wd]));
      }
      u32x4 pa;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const uint32_t lo_src = static_cast<uint32_t>(
            __builtin_amdgcn_mov_dpp(static_cast<int>(lo[wd]), 0x110 + G, 0xF, 0xF, false));
        pa[wd] = (n16 < G) ? hi[wd] : ((n16 < 2 * G) ? lo_src : 0u);
      }
      u32x4 vf[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) vf[nb] = widen8<DT>(vraw[nb][0], vraw[nb][1]);
      if (prefetch) {
        asm volatile("" ::: "memory");
        load_v(s + NW);
        asm volatile("" ::: "memory");
      }
      if (nvalid < 32) {
        // Codes past the context are stale (possibly NaN): zero them, never multiply them.
        const int keep = min(8, max(0, nvalid - tb));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) vf[nb] = keep_first8(vf[nb], keep);
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) o[nb] = mfma_f8<DT>(pa, vf[nb], o[nb]);
    };

    load_k(st);
    load_ks(st);
    load_v(st);
    load_vs(st);
    for (; st + NW < cend; st += NW) step(st, true);
    step(st, false);
  }

  l_run = group4_sum(l_run);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      if constexpr (G >= 4) {
        o[nb][jj] += __shfl_down(o[nb][jj], 16 * (G / 4));
      } else if (jj + G < 4) {
        o[nb][jj] += o[nb][jj + G];
      }
    }
  }
  float (&sO)[NW][G][D] = *reinterpret_cast<float (*)[NW][G][D]>(smem);
  float (&sM)[NW][G] = *reinterpret_cast<float (*)[NW][G]>(smem + NW * G * D);
  float (&sL)[NW][G] = *reinterpret_cast<float (*)[NW][G]>(smem + NW * G * D + NW * G);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int r = 4 * q4 + jj;
      if (r < G) sO[w][r][nb * 16 + n16] = o[nb][jj];
    }
  }
  if (q4 == 0 && n16 < G) {
    sM[w][n16] = m_run;
    sL[w][n16] = l_run;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
    const int h = idx / D;
    const int d = idx % D;
    float M = sM[0][h];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) M = fmaxf(M, sM[ww][h]);
    float acc = 0.f, lsum = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float f = fast_exp2(sM[ww][h] - M);  // waves without a step hold m = -inf -> 0
      acc += f * sO[ww][h][d];
      lsum += f * sL[ww][h];
    }
    emit_f8<DT_OUT>(a, b, g * G + h, p, nparts, d, D, M, lsum, acc);
  }
}

inline size_t align256_f8(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Validates the FP8 decode arguments and fills `a` (partition plan, workspace views, longest-first
// work order from host_lens); `wide` = 8 waves per workgroup (the single pass and partitions above
// 512 tokens), else 4.  Returns PKV_OK with empty set when there is no work (B or max_ctx 0).
inline int fp8_setup(const char* fn, Fp8Args& a, bool& wide, bool& empty, void* out, int32_t out_dtype,
                     const void* query, const void* k_cache, const void* v_cache, const void* k_scale,
                     const void* v_scale, const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                     int32_t Hq, int32_t Hkv, int32_t D, int32_t bs, int32_t max_blocks, int32_t num_blocks,
                     int32_t max_ctx, float scale, int32_t partition_size, void* workspace,
                     size_t workspace_bytes, int32_t q_dtype, const int32_t* host_lens, const void* new_k,
                     const void* new_v) {
  empty = true;
  if (q_dtype != PKV_BF16 && q_dtype != PKV_F16)
    return fail(PKV_EUNSUPPORTED, "%s: query dtype %d (bf16 or fp16)", fn, q_dtype);
  if (out_dtype != PKV_F32 && out_dtype != q_dtype)
    return fail(PKV_EINVAL, "%s: out_dtype must be PKV_F32 or the query dtype", fn);
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
  if (B == 0 || max_ctx == 0) return PKV_OK;
  if (!out || !query || !k_cache || !v_cache || !k_scale || !v_scale || !block_tables || !context_lens)
    return fail(PKV_EINVAL, "%s: NULL pointer", fn);
  int32_t part_size, max_parts;
  size_t ml_bytes = 0, need = 0;
  if (partition_size <= 0) {
    part_size = std::max(kBlock, static_cast<int32_t>(((static_cast<int64_t>(max_ctx) + kBlock - 1) / kBlock) * kBlock));
    max_parts = 1;
  } else {
    part_size = partition_size;
    max_parts = static_cast<int32_t>((static_cast<int64_t>(max_ctx) + partition_size - 1) / partition_size);
    ml_bytes = align256_f8(static_cast<size_t>(B) * Hq * max_parts * 2 * sizeof(float));
    need = ml_bytes + static_cast<size_t>(B) * Hq * max_parts * D * sizeof(float);
  }
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PKV_EINVAL, "%s: workspace of %zu bytes needed, %zu given", fn, need, workspace_bytes);
  const uintptr_t al = reinterpret_cast<uintptr_t>(query) | reinterpret_cast<uintptr_t>(k_cache) |
                       reinterpret_cast<uintptr_t>(v_cache) | reinterpret_cast<uintptr_t>(k_scale) |
                       reinterpret_cast<uintptr_t>(v_scale) | reinterpret_cast<uintptr_t>(workspace);
  if (al % 16 != 0) return fail(PKV_EINVAL, "%s: query, caches, scales and workspace must be 16-byte aligned", fn);
  if (new_k != nullptr || new_v != nullptr) {
    if (!new_k || !new_v) return fail(PKV_EINVAL, "%s: NULL new_key or new_value", fn);
    if ((reinterpret_cast<uintptr_t>(new_k) | reinterpret_cast<uintptr_t>(new_v)) % 16 != 0)
      return fail(PKV_EINVAL, "%s: new_key and new_value must be 16-byte aligned", fn);
  }
  a = Fp8Args{};
  a.out = out;
  a.q = query;
  a.k = static_cast<const uint8_t*>(k_cache);
  a.v = static_cast<const uint8_t*>(v_cache);
  a.ksc = static_cast<const float*>(k_scale);
  a.vsc = static_cast<const float*>(v_scale);
  a.tables = block_tables;
  a.lens = context_lens;
  a.part_ml = need ? static_cast<float*>(workspace) : nullptr;
  a.part_o = need ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + ml_bytes) : nullptr;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.max_blocks = max_blocks;
  a.num_blocks = num_blocks;
  a.max_parts = max_parts;
  a.part_size = part_size;
  a.scale_log2 = scale * kLog2eF8;
  if (new_k != nullptr) {
    a.new_k = new_k;
    a.new_v = new_v;
    a.k_out = const_cast<uint8_t*>(a.k);
    a.v_out = const_cast<uint8_t*>(a.v);
    a.ksc_out = const_cast<float*>(a.ksc);
    a.vsc_out = const_cast<float*>(a.vsc);
  }
  if (host_lens != nullptr && B <= kMaxOrderF8) {
    for (int i = 0; i < B; ++i) a.order[i] = i;
    std::stable_sort(a.order, a.order + B, [&](int32_t x, int32_t y) { return host_lens[x] > host_lens[y]; });
    a.num_order = B;
  }
  wide = partition_size == 0 || a.part_size > 512;
  empty = false;
  return PKV_OK;
}

}  // namespace
}  // namespace pkv
