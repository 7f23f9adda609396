// One workgroup of paged decode attention over the FP8 (E4M3) cache for a GROUP of NS sequences
// that may share cached blocks, used by the grouped FP8 decode kernel (csrc/fp8.hip).
//
// [Chapter] "Continuous batching and PagedAttention", "PagedAttention: KV cache memory": forked
// samples and requests with a common prefix point at the same physical blocks; [Notes] "Memory,
// not compute, caps the batch": a quantised cache holds more of them.  The structure is the bf16
// grouped body's (csrc/decode_group.h): the NS sequences' query heads fill the matrix columns
// (column c = sequence c / G, head c % G; NS * G is 8 or 16), a 32-token step whose two blocks are
// the same in every member's table is loaded once (codes and scales) and scored for all members,
// and a step whose blocks differ runs once per member with only that member's columns taking
// part.  Each column's arithmetic is the FP8 single-sequence body's (csrc/decode_fp8_part.h)
// operation for operation: the same steps per wave, widening, key scale inside the score, value
// scale on the weight after the softmax sum, lazy rescale, hi/lo weights and wave merge; masked
// columns only see exact no-ops.  So each sequence's output is bit for bit what
// paged_attention_decode_fp8 produces for it with the same partition size.  Codes and scales of
// tokens that some member of a pass sees must be finite (a member's zero weight meets the other
// members' values in the shared products); past every taking-part member's context, codes and
// value scales are zeroed.
#pragma once
#include "decode_fp8_part.h"

namespace pkv {
namespace {

template <int D, int G, int NS, int NW>
constexpr int fp8_group_smem_floats() {
  return NW * NS * G * D + 2 * NW * NS * G;
}

// Group grp = sequences grp * NS .. grp * NS + NS - 1 (those below B), KV head g, partition p.
template <int DT, int DT_OUT, int D, int G, int NS, int NW>
__device__ __forceinline__ void decode_fp8_group_part(const Fp8Args& a, int B, int g, int grp, int p, float* smem) {
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(NS >= 2 && NS * G <= 16, "group columns");
  constexpr int C = NS * G;          // query columns of the group
  constexpr int RT = C > 8 ? 2 : 1;  // P.V row tiles (C hi rows + C lo rows)
  constexpr int KP = D / 64;
  constexpr int KS = D / 32;
  constexpr int NB = D / 16;
  constexpr int TILE = kBlock * D;
  constexpr int kTableSteps = 32;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15;
  const int q4 = lane >> 4;
  const int pstart = p * a.part_size;

  int seq[NS], pend[NS], nparts[NS];
  // Each member's first table chunk is loaded before its length is known (its index is bounded
  // by the table row, not by the length), so the first K/V loads wait for one load, not two.
  int tab_first[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    seq[s] = grp * NS + s;
    const int32_t* row = a.tables + static_cast<int64_t>(seq[s] < B ? seq[s] : 0) * a.max_blocks;
    tab_first[s] = row[min((pstart >> 4) + lane, a.max_blocks - 1)];
  }
  int nsteps = 0;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int L = seq[s] < B ? clamp_len_f8(a, seq[s]) : 0;
    pend[s] = L > pstart ? min(pstart + a.part_size, L) : pstart;
    nparts[s] = (L + a.part_size - 1) / a.part_size;
    nsteps = max(nsteps, (pend[s] - pstart + 31) >> 5);
  }
  if (nsteps == 0) return;  // the whole workgroup leaves together

  const int ms = n16 / G;
  const int hs = n16 % G;
  int my_pend = pstart;
#pragma unroll
  for (int s = 0; s < NS; ++s) my_pend = (n16 < C && ms == s) ? pend[s] : my_pend;
  int my_seq = 0;
#pragma unroll
  for (int s = 0; s < NS; ++s) my_seq = (ms == s) ? seq[s] : my_seq;

  // Query fragments in the K loads' dimension order: k-step 2p + h holds [64p + 16 q4 + 8h, +8).
  u32x4 qf[KS];
  {
    const bool has_q = my_pend > pstart;
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           (static_cast<int64_t>(has_q ? my_seq : 0) * a.Hq + g * G + hs) * D;
#pragma unroll
    for (int pp = 0; pp < KP; ++pp) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        qf[2 * pp + hf] = has_q ? *reinterpret_cast<const u32x4*>(qrow + 64 * pp + 16 * q4 + 8 * hf)
                                : u32x4{0, 0, 0, 0};
    }
  }
  const bool k_from_b = n16 >= 8;
  const int k_in_tile = (n16 & 7) * 64 + q4 * 16;
  const bool v_from_b = q4 >= 2;
  const int v_in_tile = n16 * kBlock + (q4 & 1) * 8;
  const bool s_from_b = q4 >= 2;
  const int s_in_head = (q4 & 1) * 8;
  const int tb = 8 * q4;

  f32x4 o[RT][NB];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[rt][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float m_run = -INFINITY;
  float l_run = 0.f;

  for (int c0 = 0; c0 < nsteps; c0 += kTableSteps) {
    const int cend = min(nsteps, c0 + kTableSteps);
    int st = c0 + w;
    if (st >= cend) continue;
    const int cb0 = (pstart >> 4) + 2 * c0;
    int tab[NS], cnb[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int32_t* row = a.tables + static_cast<int64_t>(seq[s] < B ? seq[s] : 0) * a.max_blocks;
      tab[s] = clamp_blk_f8(a, c0 == 0 ? tab_first[s] : row[min(cb0 + lane, a.max_blocks - 1)]);
      cnb[s] = min(2 * kTableSteps, ((pend[s] + 15) >> 4) - cb0);
    }
    auto blocks_of = [&](int s_tab, int s_cnb, int t, int& bA, int& bB) {
      const int j = 2 * (t - c0);
      bA = __builtin_amdgcn_readlane(s_tab, j);
      bB = __builtin_amdgcn_readlane(s_tab, min(j + 1, max(s_cnb, 1) - 1));
    };
    auto head = [&](int blk) { return static_cast<int64_t>(blk) * a.Hkv + g; };
    auto plan = [&](int t, int& bA, int& bB, int& vmax) -> bool {
      bool shared = true, have = false;
      vmax = 0;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int nv = min(32, pend[s] - (pstart + t * 32));
        if (nv > 0) {
          int xA, xB;
          blocks_of(tab[s], cnb[s], t, xA, xB);
          if (!have) {
            bA = xA;
            bB = xB;
            have = true;
          } else if (xA != bA || xB != bB) {
            shared = false;
          }
          vmax = max(vmax, nv);
        }
      }
      return shared;
    };

    u32x4 kraw[2 * KP];
    u32x2 vraw[NB];
    f32x4 ksc[2], vsc[2];
    auto load_k = [&](int bA, int bB) {
      const uint8_t* kp = a.k + head(k_from_b ? bB : bA) * TILE + k_in_tile;
#pragma unroll
      for (int ss = 0; ss < 2; ++ss) {
#pragma unroll
        for (int pp = 0; pp < KP; ++pp)
          kraw[ss * KP + pp] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + (pp * 2 + ss) * 512));
      }
    };
    auto load_ks = [&](int bA, int bB) {
      const float* sp = a.ksc + head(s_from_b ? bB : bA) * kBlock + s_in_head;
      ksc[0] = *reinterpret_cast<const f32x4*>(sp);
      ksc[1] = *reinterpret_cast<const f32x4*>(sp + 4);
    };
    auto load_v = [&](int bA, int bB) {
      const uint8_t* vp = a.v + head(v_from_b ? bB : bA) * TILE + v_in_tile;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        vraw[nb] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(vp + nb * 16 * kBlock));
    };
    auto load_vs = [&](int bA, int bB) {
      const float* sp = a.vsc + head(s_from_b ? bB : bA) * kBlock + s_in_head;
      vsc[0] = *reinterpret_cast<const f32x4*>(sp);
      vsc[1] = *reinterpret_cast<const f32x4*>(sp + 4);
    };

    // One pass over step t with its codes and scales loaded: only member `only`'s columns take
    // part (every member with a token in the step when only < 0); codes and value scales are kept
    // up to vkeep tokens.  With `prefetch`, step t + NW's (blocks nA, nB) are loaded as the
    // registers free up.
    auto pass = [&](int t, int only, int vkeep, const bool prefetch, int nA, int nB) {
      const int my_nvalid = min(32, my_pend - (pstart + t * 32));
      const bool col_on = my_nvalid > 0 && (only < 0 || ms == only);
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
        load_k(nA, nB);
        asm volatile("" ::: "memory");
      }
      f32x4 s1 = {0.f, 0.f, 0.f, 0.f}, s2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s1 = mfma_f8<DT>(kf[0][ks], qf[ks], s1);
        s2 = mfma_f8<DT>(kf[1][ks], qf[ks], s2);
      }
      float sc[8];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        sc[jj] = (col_on && tb + jj < my_nvalid) ? s1[jj] * (ksc[0][jj] * a.scale_log2) : -INFINITY;
        sc[4 + jj] = (col_on && tb + 4 + jj < my_nvalid) ? s2[jj] * (ksc[1][jj] * a.scale_log2) : -INFINITY;
      }
      if (prefetch) load_ks(nA, nB);
      float bmax = sc[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) bmax = fmaxf(bmax, sc[i]);
      bmax = group4_max(bmax);
      const bool need = col_on && (bmax > m_run + kLazyRescaleLog2F8);
      if (__any(need)) {
        const float m_new = need ? bmax : m_run;
        const float alpha = need ? fast_exp2(m_run - m_new) : 1.0f;
        l_run *= alpha;
        m_run = m_new;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int r = 4 * q4 + jj;
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const float f = __shfl(alpha, RT == 1 ? r % C : rt * 8 + r % 8);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) o[rt][nb][jj] *= f;
          }
        }
      }
      float pw[8];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float pv = col_on ? fast_exp2(sc[i] - m_run) : 0.f;
        psum += pv;
        // the value scale of a token past every taking-part member's context may be stale (NaN)
        const float vs = tb + i < vkeep ? vsc[i >> 2][i & 3] : 0.f;
        pw[i] = pv * vs;
      }
      l_run += psum;
      if (prefetch) load_vs(nA, nB);
      u32x4 hi, lo;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        hi[wd] = pack2<DT>(pw[2 * wd], pw[2 * wd + 1]);
        lo[wd] = pack2<DT>(pw[2 * wd] - low_half<DT>(hi[wd]), pw[2 * wd + 1] - high_half<DT>(hi[wd]));
      }
      u32x4 pa[RT];
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        if constexpr (RT == 1) {
          const uint32_t lo_src = static_cast<uint32_t>(
              __builtin_amdgcn_mov_dpp(static_cast<int>(lo[wd]), 0x110 + C, 0xF, 0xF, false));
          pa[0][wd] = (n16 < C) ? hi[wd] : ((n16 < 2 * C) ? lo_src : 0u);
        } else {
          const uint32_t lo_src = static_cast<uint32_t>(
              __builtin_amdgcn_mov_dpp(static_cast<int>(lo[wd]), 0x118, 0xF, 0xF, false));  // row_shr:8
          const uint32_t hi_src = static_cast<uint32_t>(
              __builtin_amdgcn_mov_dpp(static_cast<int>(hi[wd]), 0x108, 0xF, 0xF, false));  // row_shl:8
          pa[0][wd] = (n16 < 8) ? hi[wd] : lo_src;
          pa[1][wd] = (n16 < 8) ? hi_src : lo[wd];
        }
      }
      u32x4 vf[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) vf[nb] = widen8<DT>(vraw[nb][0], vraw[nb][1]);
      if (prefetch) {
        asm volatile("" ::: "memory");
        load_v(nA, nB);
        asm volatile("" ::: "memory");
      }
      if (vkeep < 32) {
        const int keep = min(8, max(0, vkeep - tb));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) vf[nb] = keep_first8(vf[nb], keep);
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) o[rt][nb] = mfma_f8<DT>(pa[rt], vf[nb], o[rt][nb]);
      }
    };

    while (st < cend) {
      int cA = 0, cB = 0, cvmax = 0;
      if (plan(st, cA, cB, cvmax)) {
        load_k(cA, cB);
        load_ks(cA, cB);
        load_v(cA, cB);
        load_vs(cA, cB);
        int nA = 0, nB = 0, nvmax = 0;
        while (st + NW < cend && plan(st + NW, nA, nB, nvmax)) {
          pass(st, -1, cvmax, true, nA, nB);
          st += NW;
          cvmax = nvmax;
        }
        pass(st, -1, cvmax, false, 0, 0);
      } else {
#pragma unroll 1
        for (int s = 0; s < NS; ++s) {
          int s_pend = pend[0], s_tab = tab[0], s_cnb = cnb[0];
#pragma unroll
          for (int x = 1; x < NS; ++x) {
            if (x == s) {
              s_pend = pend[x];
              s_tab = tab[x];
              s_cnb = cnb[x];
            }
          }
          const int nv = min(32, s_pend - (pstart + st * 32));
          if (nv > 0) {
            int xA, xB;
            blocks_of(s_tab, s_cnb, st, xA, xB);
            load_k(xA, xB);
            load_ks(xA, xB);
            load_v(xA, xB);
            load_vs(xA, xB);
            pass(st, s, nv, false, 0, 0);
          }
        }
      }
      st += NW;
    }
  }

  l_run = group4_sum(l_run);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (RT == 2) {
        o[0][nb][j] += __shfl_down(o[0][nb][j], 32);
        o[1][nb][j] += __shfl_down(o[1][nb][j], 32);
      } else if constexpr (C >= 4) {
        o[0][nb][j] += __shfl_down(o[0][nb][j], 16 * (C / 4));
      } else if (j + C < 4) {
        o[0][nb][j] += o[0][nb][j + C];
      }
    }
  }

  float (&sO)[NW][C][D] = *reinterpret_cast<float (*)[NW][C][D]>(smem);
  float (&sM)[NW][C] = *reinterpret_cast<float (*)[NW][C]>(smem + NW * C * D);
  float (&sL)[NW][C] = *reinterpret_cast<float (*)[NW][C]>(smem + NW * C * D + NW * C);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 4 * q4 + j;
        if (RT == 2 ? r < 8 : r < C) sO[w][RT == 2 ? rt * 8 + r : r][nb * 16 + n16] = o[rt][nb][j];
      }
    }
  }
  if (q4 == 0 && n16 < C) {
    sM[w][n16] = m_run;
    sL[w][n16] = l_run;
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < C * D; idx += NW * 64) {
    const int c = idx / D;
    const int d = idx % D;
    const int s = c / G;
    int b = 0, np = 0;
    bool live = false;
#pragma unroll
    for (int x = 0; x < NS; ++x) {
      if (x == s) {
        b = seq[x];
        np = nparts[x];
        live = pend[x] > pstart;
      }
    }
    if (!live) continue;
    float M = sM[0][c];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) M = fmaxf(M, sM[ww][c]);
    float acc = 0.f, lsum = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float f = fast_exp2(sM[ww][c] - M);
      acc += f * sO[ww][c][d];
      lsum += f * sL[ww][c];
    }
    emit_f8<DT_OUT>(a, b, g * G + c % G, p, np, d, D, M, lsum, acc);
  }
}

}  // namespace
}  // namespace pkv
