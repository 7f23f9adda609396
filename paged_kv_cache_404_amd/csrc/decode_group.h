// One workgroup of paged decode attention for a GROUP of NS sequences that may share cached
// blocks (forked samples of one prompt, requests with a common prefix), shared by the grouped
// decode kernel (csrc/decode.hip) and the mixed decode + prefill launch (csrc/mixed.hip).
//
// [Chapter] "Continuous batching and PagedAttention", "PagedAttention: KV cache memory": several
// samples of the same answer, or conversations with a common prefix, point at the same physical
// blocks, so the prefix is stored once.  The single-sequence workgroup (decode_part.h) still reads
// a shared block once per sequence.  Here the NS sequences' query heads fill the columns of the
// Q.K matrix product (column c = sequence c / G, head c % G; NS * G <= 16), and a 32-token step
// whose two blocks are the same in every member's table is loaded once and scored for all of them.
// A step whose blocks differ between members (the private tail after the shared prefix) runs once
// per member with only that member's columns unmasked.
//
// Every column's arithmetic is the single-sequence kernel's, operation for operation: the same
// steps per wave (step s of a partition belongs to wave s % NW), the same matrix instruction and
// token order, the same lazy rescale, the hi/lo split of the weights, the same wave merge.  Matrix
// columns (and P.V rows) are independent, and masked columns only ever see exact no-ops (weights
// 0, rescale factor 1).  So each sequence's output is bit for bit what decode_mfma_part produces
// for it, whatever its group.  (K/V values must be finite: a masked column's zero weight meets the
// other members' values in P.V.)
#pragma once
#include "decode_part.h"

namespace pkv {
namespace {

// LDS of one workgroup of the body below, in floats: the waves' partial outputs, maxima and sums
// per column.
template <int D, int G, int NS, int NW>
constexpr int group_smem_floats() {
  return NW * NS * G * D + 2 * NW * NS * G;
}

// Group grp = sequences grp * NS .. grp * NS + NS - 1 (those below B), KV head g, partition p.
// No work order: rows are groups in batch order.
template <int DT, int DT_OUT, int D, int G, int NS, int NW>
__device__ __forceinline__ void decode_group_part(const DecodeArgs& a, int B, int g, int grp, int p, float* smem) {
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(NS >= 2 && NS * G <= 16, "group columns");
  constexpr int C = NS * G;           // query columns of the group
  constexpr int RT = C > 8 ? 2 : 1;   // P.V row tiles (C hi rows + C lo rows)
  constexpr int KS = D / 32;
  constexpr int NB = D / 16;
  constexpr int TILE = kBlock * D;
  constexpr int kTableSteps = 32;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n16 = lane & 15;
  const int q4 = lane >> 4;
  const int pstart = p * a.part_size;

  // Members: sequence, end of this partition (pstart when the member has no token in it), count
  // of partitions.  Uniform values.
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
    const int L = seq[s] < B ? clamp_len(a, seq[s]) : 0;
    pend[s] = L > pstart ? min(pstart + a.part_size, L) : pstart;
    nparts[s] = (L + a.part_size - 1) / a.part_size;
    nsteps = max(nsteps, (pend[s] - pstart + 31) >> 5);
  }
  if (nsteps == 0) return;  // the whole workgroup leaves together

  // This lane's column: member ms, head hs; my_pend = that member's partition end.
  const int ms = n16 / G;
  const int hs = n16 % G;
  int my_pend = pstart;
#pragma unroll
  for (int s = 0; s < NS; ++s) my_pend = (n16 < C && ms == s) ? pend[s] : my_pend;
  int my_seq = 0;
#pragma unroll
  for (int s = 0; s < NS; ++s) my_seq = (ms == s) ? seq[s] : my_seq;

  const uint16_t* __restrict__ kc = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ vc = static_cast<const uint16_t*>(a.v);

  // Q^T fragments: lane (column n16, group q4) holds Q[member][head][ks*32 + 8*q4 .. +8].
  u32x4 qf[KS];
  {
    const bool has_q = my_pend > pstart;
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           (static_cast<int64_t>(has_q ? my_seq : 0) * a.Hq + g * G + hs) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = has_q ? *reinterpret_cast<const u32x4*>(qrow + ks * 32 + q4 * 8) : u32x4{0, 0, 0, 0};
  }

  // Token order of a step and tile offsets: as in decode_mfma_part.
  const int k_in_tile = (q4 * 8 + (n16 & 7)) * 8;
  const bool k_from_b = n16 >= 8;
  const bool v_from_b = q4 >= 2;
  const int v_in_tile = (q4 & 1) * D * 8 + n16 * 8;
  const int tb = 8 * q4;

  f32x4 o[RT][NB];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) o[rt][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float m_run = -INFINITY;  // this lane's column: reference maximum (log2 domain)
  float l_run = 0.f;        // this lane's share of the column's sum of weights

  for (int c0 = 0; c0 < nsteps; c0 += kTableSteps) {
    const int cend = min(nsteps, c0 + kTableSteps);
    int st = c0 + w;
    if (st >= cend) continue;
    const int cb0 = (pstart >> 4) + 2 * c0;  // first block of this table chunk
    int tab[NS], cnb[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int32_t* row = a.tables + static_cast<int64_t>(seq[s] < B ? seq[s] : 0) * a.max_blocks;
      tab[s] = clamp_blk(a, c0 == 0 ? tab_first[s] : row[min(cb0 + lane, a.max_blocks - 1)]);
      cnb[s] = min(2 * kTableSteps, ((pend[s] + 15) >> 4) - cb0);
    }

    // Block ids of member s's two blocks in step t (a lone last block pairs with itself).
    auto blocks_of = [&](int s_tab, int s_cnb, int t, int& bA, int& bB) {
      const int j = 2 * (t - c0);
      bA = __builtin_amdgcn_readlane(s_tab, j);
      bB = __builtin_amdgcn_readlane(s_tab, min(j + 1, max(s_cnb, 1) - 1));
    };
    auto tile = [&](int blk) { return (static_cast<int64_t>(blk) * a.Hkv + g) * TILE; };
    // Step t is shared when every member with a token in it reads the same two blocks; then
    // (bA, bB) are those blocks and vmax the most tokens any member has in the step.
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

    u32x4 kf[2 * KS], vf[NB];
    auto load_k = [&](int bA, int bB) {
      const uint16_t* kp = kc + tile(k_from_b ? bB : bA) + k_in_tile;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        kf[ks] = *reinterpret_cast<const u32x4*>(kp + (2 * ks) * 256);
        kf[KS + ks] = *reinterpret_cast<const u32x4*>(kp + (2 * ks + 1) * 256);
      }
    };
    auto load_v = [&](int bA, int bB) {
      const uint16_t* vp = vc + tile(v_from_b ? bB : bA) + v_in_tile;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) vf[nb] = *reinterpret_cast<const u32x4*>(vp + nb * 16 * 8);
    };

    // One pass over step t with the K/V registers loaded: only member `only`'s columns take part
    // (all members with a token in the step when only < 0); V is kept up to vkeep tokens.  With
    // `prefetch`, step t + NW's K/V (blocks nA, nB) are loaded as the registers free up.
    auto pass = [&](int t, int only, int vkeep, const bool prefetch, int nA, int nB) {
      const int my_nvalid = min(32, my_pend - (pstart + t * 32));
      const bool col_on = my_nvalid > 0 && (only < 0 || ms == only);
      f32x4 s1 = {0.f, 0.f, 0.f, 0.f}, s2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s1 = mfma16x16x32<DT>(kf[ks], qf[ks], s1);
        s2 = mfma16x16x32<DT>(kf[KS + ks], qf[ks], s2);
      }
      if (prefetch) {
        asm volatile("" ::: "memory");
        load_k(nA, nB);
        asm volatile("" ::: "memory");
      }
      float sc[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sc[j] = (col_on && tb + j < my_nvalid) ? s1[j] * a.scale_log2 : -INFINITY;
        sc[4 + j] = (col_on && tb + 4 + j < my_nvalid) ? s2[j] * a.scale_log2 : -INFINITY;
      }
      float bmax = sc[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) bmax = fmaxf(bmax, sc[i]);
      bmax = group4_max(bmax);

      const bool need = col_on && (bmax > m_run + kLazyRescaleLog2);
      if (__any(need)) {
        const float m_new = need ? bmax : m_run;
        const float alpha = need ? fast_exp2(m_run - m_new) : 1.0f;
        l_run *= alpha;
        m_run = m_new;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 4 * q4 + j;
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const float f = __shfl(alpha, RT == 1 ? r % C : rt * 8 + r % 8);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) o[rt][nb][j] *= f;
          }
        }
      }

      float pv[8];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pv[i] = col_on ? fast_exp2(sc[i] - m_run) : 0.f;
        psum += pv[i];
      }
      l_run += psum;

      u32x4 hi, lo;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        hi[wd] = pack2<DT>(pv[2 * wd], pv[2 * wd + 1]);
        lo[wd] = pack2<DT>(pv[2 * wd] - low_half<DT>(hi[wd]), pv[2 * wd + 1] - high_half<DT>(hi[wd]));
      }
      // P rows: one tile holds the C hi rows then the C lo rows (C <= 8); with 16 columns, tile 0
      // holds columns 0..7 (hi rows 0..7, lo rows 8..15) and tile 1 columns 8..15 alike.
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
      if (vkeep < 32) {
        // Tokens past every taking-part member's context are stale (possibly NaN): zero them.
        const int keep = min(8, max(0, vkeep - tb));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) vf[nb] = keep_first(vf[nb], keep);
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) o[rt][nb] = mfma16x16x32<DT>(pa[rt], vf[nb], o[rt][nb]);
      }
      if (prefetch) {
        asm volatile("" ::: "memory");
        load_v(nA, nB);
        asm volatile("" ::: "memory");
      }
    };

    // Runs of shared steps go as in decode_mfma_part (loads of the next step issued during the
    // current one, the run's last step peeled); a step whose blocks differ between members runs
    // once per member with a token in it (a rolled loop; the member's table register and end
    // are picked by selects).
    while (st < cend) {
      int cA = 0, cB = 0, cvmax = 0;
      if (plan(st, cA, cB, cvmax)) {
        load_k(cA, cB);
        load_v(cA, cB);
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
            load_v(xA, xB);
            pass(st, s, nv, false, 0, 0);
          }
        }
      }
      st += NW;
    }
  }

  // Per-column sums over the four lane groups; fold every column's lo row into its hi row.
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
    emit<DT_OUT>(a, b, g * G + c % G, p, np, d, D, M, lsum, acc);
  }
}

}  // namespace
}  // namespace pkv
